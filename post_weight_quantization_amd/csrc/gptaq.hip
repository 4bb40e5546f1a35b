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
// Per 128-column block: a panel kernel sweeps the block in registers
// (16 lanes per row, 8 columns per lane; U's diagonal block sits in LDS,
// permuted so each lane reads its 8 entries of row p as two 16-byte loads),
// writes codes, W^ and the scaled errors E; then the lazy trailing update
// W_bar[:, >blk] -= E U_{blk, >blk} runs as an fp32 MFMA GEMM.
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int BK = 128;  // block / group width

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

// The column sweep of one 128-column block.
// Thread t: row r = blockIdx.x * 16 + t / 16, lane-in-row c = t % 16, holding
// columns blk0 + 16 j + c (j = 0..7) of W_bar.
__global__ __launch_bounds__(256) void panel_kernel(const float* __restrict__ Wbar,
                                                    const float* __restrict__ U,
                                                    const float* __restrict__ Z, float* Wout,
                                                    uint8_t* codes, float* E, float* scale,
                                                    float* zero, int64_t d_out, int64_t n,
                                                    int64_t blk0, int ngroups, int grouped,
                                                    float maxq) {
  __shared__ float Us[BK * BK];  // Us[p][c][j] = U[blk0 + p][blk0 + 16 j + c]
  __shared__ float uinv[BK];
  const int t = threadIdx.x;
  // stage U's diagonal block (coalesced reads, permuted writes)
  for (int e = t; e < BK * BK; e += 256) {
    const int p = e >> 7, m = e & 127;
    Us[p * BK + (m & 15) * 8 + (m >> 4)] = U[(blk0 + p) * n + blk0 + m];
  }
  if (t < BK) uinv[t] = 1.f / U[(blk0 + t) * n + blk0 + t];

  const int c = t & 15;
  const int64_t row = int64_t(blockIdx.x) * 16 + (t >> 4);
  const bool valid = row < d_out;
  const int64_t rr = valid ? row : d_out - 1;
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = Wbar[rr * n + blk0 + 16 * j + c];

  float sc, zr;
  if (grouped) {
    // grid of this group from the working values minus the in-group P terms
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = w[j];
      if (Z) v -= Z[rr * n + blk0 + 16 * j + c];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
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

  float q_out[8], w_out[8], e_out[8];
  const int base_lane = (threadIdx.x & 63) & ~15;
#pragma unroll
  for (int p = 0; p < BK; ++p) {
    const int j0 = p >> 4;
    const int c0 = p & 15;
    const float x = w[j0];
    const float q = fminf(fmaxf(rintf(x * isc) + zr, 0.f), maxq);
    const float wq = sc * (q - zr);
    float e = (x - wq) * uinv[p];
    e = __shfl(e, base_lane + c0, 64);
    if (c == c0) {
      q_out[j0] = q;
      w_out[j0] = wq;
      e_out[j0] = e;
    }
    const float* up = Us + p * BK + c * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (16 * j + 15 <= p) continue;  // every column of this register is finished
      w[j] -= e * up[j];
    }
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = blk0 + 16 * j + c;
      codes[row * n + col] = uint8_t(q_out[j]);
      Wout[row * n + col] = w_out[j];
      E[row * BK + 16 * j + c] = e_out[j];
    }
  }
}

}  // namespace

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
  ar.take<float>(size_t(d_out) * BK); // E
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
  float* E = ws.take<float>(size_t(d_out) * BK);
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
  const int64_t nblk = n / BK;
  for (int64_t b = 0; b < nblk; ++b) {
    const int64_t blk0 = b * BK;
    panel_kernel<<<unsigned(cdiv(d_out, 16)), 256, 0, s>>>(Wbar, U, Z, W, codes, E, scale, zero,
                                                           d_out, n, blk0, ngroups, group ? 1 : 0,
                                                           maxq);
    KQ_HIP(hipGetLastError());
    const int64_t rest = n - blk0 - BK;
    if (rest > 0) {
      // W_bar[:, blk0+BK:] -= E U[blk0:blk0+BK, blk0+BK:]
      GemmArgs gt = gemm_args(E, BK, U + blk0 * n + blk0 + BK, n, Wbar + blk0 + BK, n, d_out, rest,
                              BK, -1.f, 1.f, 0);
      KQ_TRY(gemm_f32(gt, s));
    }
  }
  return KQ_OK;
}

}  // namespace kq
