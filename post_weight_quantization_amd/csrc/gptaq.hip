// Stage 4: the GPTAQ column sweep and its asymmetric correction P.
//
// KronQ summary (hyper.ai), Method: after quantizing column p,
//   dW_{:, p+1:} = -delta_p [H_X^-1]_{p, p+1:} + W_{:, p} P_{p, p+1:},
// delta_p the scaled rounding error, P the GPTAQ asymmetric correction. With
// U^T U = (H + delta I)^-1 the inverse row is U_{p, p+1:} and
// delta_p = (w_p - w^_p) / U_pp. P (not written out on the pages) is read as
// P = triu_1(D U^T) U, whose row p equals D_{p,F} (H_FF)^-1 — the
// least-squares compensation of the fixed column's input drift. The gist.science
// explainer (Metodologia, Proposition 1) notes that H_G cancels from the update.
//
// Because P is strictly upper and W_{:, p} is the ORIGINAL (processed) W0,
// the P terms reaching column j sum to (W0 P)_j whatever the order, so the
// sweep runs plain GPTQ on W_bar = W0 + W0 P (one fp32 MFMA GEMM, P strictly
// upper). With per-group grids computed when the sweep reaches a group, the
// in-group part of W0 P must not yet be present at that moment: the grid is
// taken from W_bar - Z with Z = W0 blockdiag_128(P) (a batched GEMM).
//
// Per 128-column block a panel kernel sweeps the block in registers (16 lanes
// per row, 8 columns per lane, U's diagonal block in LDS) and writes codes,
// W^ and the scaled errors E. The lazy update W_bar[:, >blk] -= E U_{blk,>blk}
// runs as fp32 MFMA GEMMs, grouped in 512-column superblocks so the far part
// of W_bar is read and written once per four panels.
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int BK = 128;  // block / group width
constexpr int64_t SB = 512;  // superblock of the lazy trailing updates

// Grid per output channel (fp32): lo = min(row, 0), hi = max(row, 0),
// [-1, 1] for an all-zero row, scale = (hi - lo) / maxq, zero = rint(-lo / scale).
__global__ __launch_bounds__(256) void grid_rows_kernel(const float* W, int64_t rows, int64_t cols,
                                                        float maxq, float* scale, float* zero) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* p = W + row * cols;
  float lo = 0.f, hi = 0.f;
  for (int64_t c = 4 * lane; c < cols; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(p + c);
    lo = fminf(lo, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
    hi = fmaxf(hi, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if (lane == 0) {
    if (lo == hi) {
      lo = -1.f;
      hi = 1.f;
    }
    const float sc = (hi - lo) / maxq;
    scale[row] = sc;
    zero[row] = rintf(-lo / sc);
  }
}

// The column sweep of one 128-column block, for PR = 16 rows per workgroup.
// Lane l of wave w: row row0 + 4 w + l / 16, position c = l % 16 in its group
// of 16 lanes, holding columns blk0 + 8 c + j (j = 0..7) in registers. The
// sweep runs an outer loop over the owning position c0 (not unrolled, which
// keeps the code small enough for the instruction cache) and 8 unrolled steps
// inside. Step p = 8 c0 + j0: every lane rounds its candidate w[j0]; the
// owner's scaled error reaches all 16 lanes of the row through a sum of the
// masked errors with four DPP steps (quad_perm, quad_perm, row_half_mirror,
// row_mirror), so the serial path has no LDS round trip; each lane then
// applies it to its columns with U row p from LDS (diagonal and below stored
// as zeros, each lane's 8 entries as two float4). The owner keeps its errors
// and codes in registers; every lane writes its 8 columns of W^, E and the
// codes straight to memory at the end.
constexpr int PR = 16;
constexpr int NPOS = 16;            // lanes per row
constexpr int CPL = BK / NPOS;      // columns per lane
constexpr int UROW = BK;            // floats per staged U row

// v + (v of another lane); with bound_ctrl set the move can fold into the
// add as a DPP source operand (one instruction per level)
__device__ inline float dpp_add(float v, int ctrl_sel) {
  switch (ctrl_sel) {
    case 0:  // quad_perm [1,0,3,2]
      return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
    case 1:  // quad_perm [2,3,0,1]
      return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
    case 2:  // row_half_mirror: lane i <-> 7 - i within each 8 lanes
      return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
    default:  // row_mirror: lane i <-> 15 - i within each 16 lanes
      return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
  }
}

__device__ inline float group16_sum(float v) {
  v = dpp_add(v, 0);
  v = dpp_add(v, 1);
  v = dpp_add(v, 2);
  return dpp_add(v, 3);
}

constexpr size_t PANEL_LDS = sizeof(float) * (size_t(BK) * UROW + BK);

__global__ __launch_bounds__(256) void panel_kernel(const float* __restrict__ Wbar,
                                                    const float* __restrict__ U,
                                                    const float* __restrict__ Z, float* Wout,
                                                    uint8_t* codes, float* E, int64_t ldE,
                                                    float* scale, float* zero, int64_t d_out,
                                                    int64_t n, int64_t blk0, int ngroups,
                                                    int grouped, float maxq) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* Us = sm;                 // [p][m] = U[blk0 + p][blk0 + m] if m > p, else 0
  float* uinv = Us + BK * UROW;   // 1 / U_pp
  const int t = threadIdx.x;
  {
    // U's diagonal block: 16 float4 loads per thread, all in flight together
    constexpr int NV = BK * BK / 4 / 256;
    float4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e4 = t + 256 * k;
      const int p = e4 >> 5, m = (e4 & 31) * 4;
      v[k] = *reinterpret_cast<const float4*>(U + (blk0 + p) * n + blk0 + m);
    }
    const float ud = t < BK ? U[(blk0 + t) * n + blk0 + t] : 1.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e4 = t + 256 * k;
      const int p = e4 >> 5, m = (e4 & 31) * 4;
      float4 x = v[k];
      x.x = m > p ? x.x : 0.f;
      x.y = m + 1 > p ? x.y : 0.f;
      x.z = m + 2 > p ? x.z : 0.f;
      x.w = m + 3 > p ? x.w : 0.f;
      *reinterpret_cast<float4*>(Us + p * UROW + m) = x;
    }
    if (t < BK) uinv[t] = 1.f / ud;
  }

  const int lane = t & 63;
  const int c = lane & (NPOS - 1);
  const int rloc = 4 * (t >> 6) + (lane >> 4);
  const int64_t row = int64_t(blockIdx.x) * PR + rloc;
  const bool valid = row < d_out;
  const int64_t rr = valid ? row : d_out - 1;
  const float* wsrc = Wbar + rr * n + blk0 + CPL * c;
  float w[CPL];
#pragma unroll
  for (int j = 0; j < CPL; j += 4) {
    const float4 v = *reinterpret_cast<const float4*>(wsrc + j);
    w[j] = v.x;
    w[j + 1] = v.y;
    w[j + 2] = v.z;
    w[j + 3] = v.w;
  }

  float sc, zr;
  if (grouped) {
    // grid of this group from the working values minus the in-group P terms
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float v = w[j];
      if (Z) v -= Z[rr * n + blk0 + CPL * c + j];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int o = 1; o < NPOS; o <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    if (lo == hi) {
      lo = -1.f;
      hi = 1.f;
    }
    sc = (hi - lo) / maxq;
    zr = rintf(-lo / sc);
    if (valid && c == 0) {
      const int64_t g = blk0 / BK;
      scale[row * ngroups + g] = sc;
      zero[row * ngroups + g] = zr;
    }
  } else {
    sc = scale[rr];
    zr = zero[rr];
  }
  const float isc = 1.f / sc;
  __syncthreads();

  // 1 / U_pp and the superdiagonal U_{p,p+1} of this lane's own 8 columns:
  // only the lane owning column p uses them, and they stay in registers so
  // the dependent chain of a step (quantize -> scaled error -> row sum ->
  // next candidate) never waits for LDS
  float uiv[CPL], sup[CPL - 1];
#pragma unroll
  for (int j = 0; j < CPL; j += 4) {
    const float4 v = *reinterpret_cast<const float4*>(uinv + CPL * c + j);
    uiv[j] = v.x;
    uiv[j + 1] = v.y;
    uiv[j + 2] = v.z;
    uiv[j + 3] = v.w;
  }
#pragma unroll
  for (int j = 0; j < CPL - 1; ++j) sup[j] = Us[(CPL * c + j) * UROW + CPL * c + j + 1];
  // U row p for this lane (8 entries), fetched one step ahead
  auto fetch = [&](int p, float (&u)[CPL]) {
    const float* up = Us + p * UROW + CPL * c;
#pragma unroll
    for (int k4 = 0; k4 < CPL / 4; ++k4) {
      const float4 v = *reinterpret_cast<const float4*>(up + 4 * k4);
      u[4 * k4] = v.x;
      u[4 * k4 + 1] = v.y;
      u[4 * k4 + 2] = v.z;
      u[4 * k4 + 3] = v.w;
    }
  };
  float ua[CPL], ub[CPL];
  float eown[CPL];     // this lane's scaled errors (set when it owns the column)
  uint32_t qown[2] = {0u, 0u};  // this lane's 8 codes, 4 per word
  fetch(0, ua);
#pragma unroll 1
  for (int c0 = 0; c0 < NPOS; ++c0) {
    const bool own = c == c0;
#pragma unroll
    for (int j0 = 0; j0 < CPL; ++j0) {
      const int p = CPL * c0 + j0;
      float(&ucur)[CPL] = (j0 & 1) ? ub : ua;
      float(&unxt)[CPL] = (j0 & 1) ? ua : ub;
      // zero on the lanes not owning column p, so their scaled error is 0
      // without a select on the dependent chain
      const float ui = own ? uiv[j0] : 0.f;
      if (p + 1 < BK) fetch(p + 1, unxt);
      const float x = w[j0];
      const float q = __builtin_amdgcn_fmed3f(rintf(x * isc) + zr, 0.f, maxq);
      const float wq = sc * (q - zr);
      const float el = (x - wq) * ui;
      const float e = group16_sum(el);
      if (own) {
        w[j0] = wq;
        eown[j0] = el;
        qown[j0 >> 2] |= uint32_t(q) << (8 * (j0 & 3));
      }
      // the owner's next candidate from the register superdiagonal, then
      // the rest of the row from the LDS copy of U row p
      if (j0 + 1 < CPL) w[j0 + 1] -= e * (own ? sup[j0] : 0.f);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        if (j == j0 + 1) w[j] -= e * (own ? 0.f : ucur[j]);
        else w[j] -= e * ucur[j];
      }
    }
  }
  // every lane owned its 8 columns once: W^, E and the codes go straight out
  if (valid) {
    float* wo = Wout + row * n + blk0 + CPL * c;
    float* eo = E + row * ldE + CPL * c;
#pragma unroll
    for (int j = 0; j < CPL; j += 4) {
      *reinterpret_cast<float4*>(wo + j) = make_float4(w[j], w[j + 1], w[j + 2], w[j + 3]);
      *reinterpret_cast<float4*>(eo + j) = make_float4(eown[j], eown[j + 1], eown[j + 2], eown[j + 3]);
    }
    *reinterpret_cast<uint2*>(codes + row * n + blk0 + CPL * c) = make_uint2(qown[0], qown[1]);
  }
}

}  // namespace

kq_status grid_rows(const float* W, int64_t rows, int64_t cols, float maxq, float* scale,
                    float* zero, hipStream_t s) {
  if (rows <= 0) return KQ_OK;
  grid_rows_kernel<<<unsigned(cdiv(rows, 4)), 256, 0, s>>>(W, rows, cols, maxq, scale, zero);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

size_t formp_ws_bytes(int64_t n) { return 0; }

kq_status formp_run(const float* D, const float* U, int64_t n, float* P, Arena& ws, hipStream_t s) {
  // T = triu_1(D U^T) into P's buffer, then P = T U needs T intact: use a temporary.
  float* T = ws.take<float>(size_t(n) * n);
  if (!T) return fail(KQ_ERR_WORKSPACE, "form_p: workspace too small");
  KQ_TRY(fill_f32(T, n * n, 0.f, s));
  // op(B)[k][j] = U[j][k], zero for k < j
  GemmArgs g1 = gemm_args(D, n, U, n, T, n, n, n, n, 1.f, 0.f, G_TRANS_B | G_B_LOWER | G_OUT_SUPPER);
  KQ_TRY(gemm_f32(g1, s));
  KQ_TRY(fill_f32(P, n * n, 0.f, s));
  GemmArgs g2 = gemm_args(T, n, U, n, P, n, n, n, n, 1.f, 0.f,
                          G_A_SUPPER | G_B_UPPER | G_OUT_SUPPER | G_ORDER_DIAG);
  KQ_TRY(gemm_f32(g2, s));
  return KQ_OK;
}

size_t gptaq_ws_bytes(int64_t d_out, int64_t d_in, int group, bool has_d) {
  Arena ar{nullptr, 0, 0};
  const int64_t n = d_in;
  ar.take<float>(size_t(d_out) * n);  // W_bar
  ar.take<float>(size_t(d_out) * SB); // E (one superblock)
  if (has_d) {
    ar.take<float>(size_t(n) * n);    // P
    ar.take<float>(size_t(n) * n);    // T (inside form_p)
    if (group) ar.take<float>(size_t(d_out) * n);  // Z
  }
  return ar.used;
}

kq_status gptaq_run(float* W, const float* U, const float* D, int64_t d_out, int64_t d_in, int bits,
                    int group, uint8_t* codes, float* scale, float* zero, Arena& ws, hipStream_t s) {
  const int64_t n = d_in;
  const float maxq = float((1 << bits) - 1);
  float* Wbar = ws.take<float>(size_t(d_out) * n);
  float* E = ws.take<float>(size_t(d_out) * SB);
  if (!Wbar || !E) return fail(KQ_ERR_WORKSPACE, "gptaq_quantize: workspace too small");
  float* Z = nullptr;

  if (!group) {
    grid_rows_kernel<<<unsigned(cdiv(d_out, 4)), 256, 0, s>>>(W, d_out, n, maxq, scale, zero);
    KQ_HIP(hipGetLastError());
  }
  if (D) {
    float* P = ws.take<float>(size_t(n) * n);
    if (!P) return fail(KQ_ERR_WORKSPACE, "gptaq_quantize: workspace too small");
    KQ_TRY(formp_run(D, U, n, P, ws, s));
    // W_bar = W0 + W0 P   (op(B) = P strictly upper: zero for k >= n)
    GemmArgs gf = gemm_args(W, n, P, n, Wbar, n, d_out, n, n, 1.f, 1.f, G_B_UPPER | G_ORDER_NDESC);
    gf.Cin = W;
    KQ_TRY(gemm_f32(gf, s));
    if (group) {
      Z = ws.take<float>(size_t(d_out) * n);
      if (!Z) return fail(KQ_ERR_WORKSPACE, "gptaq_quantize: workspace too small");
      // Z[:, blk] = W0[:, blk] P[blk, blk] for every diagonal block
      GemmArgs gz = gemm_args(W, n, P, n, Z, n, d_out, BK, BK, 1.f, 0.f, G_B_UPPER);
      gz.batch = int(n / BK);
      gz.strideA = BK;
      gz.strideB = BK * n + BK;
      gz.strideC = BK;
      KQ_TRY(gemm_f32(gz, s));
    }
  } else {
    KQ_HIP(hipMemcpyAsync(Wbar, W, size_t(d_out) * n * sizeof(float), hipMemcpyDeviceToDevice, s));
  }

  const int ngroups = group ? int(n / BK) : 1;
  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(panel_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(PANEL_LDS)));
  // Lazy updates in superblocks of SB columns: after each panel only the rest
  // of its superblock is updated (K = 128); the columns beyond the superblock
  // take one update with K = SB once all its panels are done.
  for (int64_t s0 = 0; s0 < n; s0 += SB) {
    const int64_t s1 = std::min(s0 + SB, n);
    for (int64_t b0 = s0; b0 < s1; b0 += BK) {
      panel_kernel<<<unsigned(cdiv(d_out, PR)), 256, PANEL_LDS, s>>>(
          Wbar, U, Z, W, codes, E + (b0 - s0), SB, scale, zero, d_out, n, b0, ngroups,
          group ? 1 : 0, maxq);
      KQ_HIP(hipGetLastError());
      const int64_t near = s1 - b0 - BK;
      if (near > 0) {
        GemmArgs gt = gemm_args(E + (b0 - s0), SB, U + b0 * n + b0 + BK, n, Wbar + b0 + BK, n, d_out,
                                near, BK, -1.f, 1.f, 0);
        KQ_TRY(gemm_f32(gt, s));
      }
    }
    const int64_t far = n - s1;
    if (far > 0) {
      GemmArgs gt = gemm_args(E, SB, U + s0 * n + s1, n, Wbar + s1, n, d_out, far, s1 - s0, -1.f,
                              1.f, 0);
      // the first superblock's update is the largest lazy GEMM: the one the
      // kernel-event hook brackets
      if (s0 == 0) KQ_TRY(mark_kernel(KQ_OP_GPTAQ_QUANTIZE, 0, s));
      KQ_TRY(gemm_f32(gt, s));
      if (s0 == 0) KQ_TRY(mark_kernel(KQ_OP_GPTAQ_QUANTIZE, 1, s));
    }
  }
  return KQ_OK;
}

}  // namespace kq
