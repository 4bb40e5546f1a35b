// Internal declarations shared by the kernels and the C ABI of libkq.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstddef>

#include "../../include/kq.h"

namespace kq {

// ---------------------------------------------------------------- errors
kq_status fail(kq_status st, const char* fmt, ...);
kq_status hip_fail(hipError_t e, const char* where);
void clear_error();

// measurement hook: records the caller's event (edge 0: start, 1: stop) for
// `op` on stream s, if one is set on this thread
kq_status mark_kernel(kq_op op, int edge, hipStream_t s);

#define KQ_HIP(expr)                                        \
  do {                                                      \
    hipError_t _e = (expr);                                 \
    if (_e != hipSuccess) return ::kq::hip_fail(_e, #expr); \
  } while (0)

#define KQ_TRY(expr)                      \
  do {                                    \
    kq_status _s = (expr);                \
    if (_s != KQ_OK) return _s;           \
  } while (0)

// ------------------------------------------------------- workspace carving
struct Arena {
  char* base;
  size_t cap;
  size_t used;
  template <class T>
  T* take(size_t count) {
    size_t off = (used + 255) & ~size_t(255);
    size_t need = off + count * sizeof(T);
    if (base == nullptr) {  // sizing pass
      used = need;
      return nullptr;
    }
    if (need > cap) return nullptr;
    used = need;
    return reinterpret_cast<T*>(base + off);
  }
};

// ------------------------------------------------------------- fp32 GEMM
// C = alpha * op(A) op(B) + beta * Cin, op(A) M x K, op(B) K x N, row-major.
enum GemmFlag : uint32_t {
  G_TRANS_A = 1u << 0,      // A stored K x M
  G_TRANS_B = 1u << 1,      // B stored N x K
  G_A_UPPER = 1u << 2,      // op(A)[m][k] = 0 for k < m  (masked at load)
  G_A_LOWER = 1u << 3,      // op(A)[m][k] = 0 for k > m
  G_B_UPPER = 1u << 4,      // op(B)[k][n] = 0 for k > n
  G_B_LOWER = 1u << 5,      // op(B)[k][n] = 0 for k < n
  G_OUT_LOWER = 1u << 6,    // write only m >= n (tiles above skipped)
  G_OUT_UPPER = 1u << 7,    // write only n >= m
  G_OUT_SUPPER = 1u << 8,   // write only n > m
  G_A_SUPPER = 1u << 9,     // op(A)[m][k] = 0 for k <= m
  // tile order (longest K range first when operands are triangular)
  G_ORDER_NDESC = 1u << 12,  // column tiles in descending order
  G_ORDER_MDESC = 1u << 13,  // row tiles in descending order
  G_ORDER_DIAG = 1u << 14,   // by (column tile - row tile), descending
  G_ORDER_NASC = 1u << 18,   // column tiles in ascending order
  // C aliases A (in place): every tile must span all N columns so that it
  // reads its rows of A before any tile writes them (requires N <= 128)
  G_C_ALIASES_A = 1u << 15,
  // skip output tiles that start before column (G_OUT_NSTART) or row
  // (G_OUT_MSTART) ostart + batch * ostart_ofs (a multiple of the tile)
  G_OUT_NSTART = 1u << 16,
  G_OUT_MSTART = 1u << 17,
};

struct GemmArgs {
  const float* A;
  const float* B;
  const float* Cin;  // may equal C; ignored when beta == 0
  float* C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t strideA, strideB, strideC;  // per batch (blockIdx.z)
  int64_t kofs;                       // per-batch offset added to k for the triangle masks
  int64_t kbase;                      // offset added to k for the triangle masks of every batch
  int64_t ostart, ostart_ofs;         // first output column / row (G_OUT_NSTART / G_OUT_MSTART)
  int batch;
  float alpha, beta;
  uint32_t flags;
};

kq_status gemm_f32(const GemmArgs& g, hipStream_t s);
// tile of later gemm_f32 calls on this thread: 0 by shape, 64, 128 or 256 forced
void set_gemm_tile(int tile);
GemmArgs gemm_args(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                   int64_t M, int64_t N, int64_t K, float alpha, float beta, uint32_t flags);

// ------------------------------------------------------------ utilities
kq_status fill_f32(float* p, int64_t n, float v, hipStream_t s);
// Copies `bytes` (at most 64) of device memory to the host once the stream's
// earlier work is done: through a pinned per-thread buffer, polling the
// stream.
kq_status read_to_host(void* dst, const void* src, size_t bytes, hipStream_t s);
kq_status fill_2d(float* p, int64_t rows, int64_t cols, int64_t ld, float v, hipStream_t s);

// ------------------------------------------------------------ covariance
size_t cov_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out, kq_dtype dt, bool hx, bool d, bool hg);
kq_status cov_run(const void* X, const void* Xq, const void* G, kq_dtype dt, int64_t n_tok,
                  int64_t d_in, int64_t d_out, float alpha, float beta, float* HX, float* D,
                  float* HG, Arena& ws, hipStream_t s);

// ------------------------------------------------------------------ BiIP
size_t biip_ws_bytes(int64_t d_out, int64_t d_in);
kq_status biip_run(float* W, float* HX, float* D, float* HG, int64_t d_out, int64_t d_in,
                   const int8_t* si, const int8_t* so, int64_t bi, int64_t bo, float* s_x,
                   float* s_g, Arena& ws, hipStream_t s);
kq_status fwht_rows(float* M, int64_t rows, int64_t cols, int64_t blk, const float* rowf,
                    const float* colf, float gain, hipStream_t s);
kq_status fwht_cols(float* M, int64_t rows, int64_t cols, int64_t blk, hipStream_t s);

// --------------------------------------------------------- sensitivity
kq_status diag_sum(const float* H, int64_t n, double* out_dev, hipStream_t s);

// ------------------------------------------------------------- Cholesky
size_t chol_ws_bytes(int64_t n);
kq_status chol_inv_run(const float* H, int64_t n, float damp, float* U, int32_t* info,
                       Arena& ws, hipStream_t s);

// ----------------------------------------------------------------- GPTAQ
size_t formp_ws_bytes(int64_t n);
kq_status formp_run(const float* D, const float* U, int64_t n, float* P, Arena& ws, hipStream_t s);
size_t gptaq_ws_bytes(int64_t d_out, int64_t d_in, int group, bool has_d);
kq_status gptaq_run(float* W, const float* U, const float* D, int64_t d_out, int64_t d_in,
                    int bits, int group, uint8_t* codes, float* scale, float* zero, Arena& ws,
                    hipStream_t s);

// ------------------------------------------------- rounding with output feedback
size_t yaqa_ws_bytes(int64_t d_out, int64_t d_in, bool has_d);
kq_status yaqa_run(float* W, const float* U_in, const float* U_out, const float* D, int64_t d_out,
                   int64_t d_in, int bits, uint8_t* codes, float* scale, float* zero, Arena& ws,
                   hipStream_t s);
// per-row grid of the sweeps (rows x cols, row stride cols, cols % 4 == 0)
kq_status grid_rows(const float* W, int64_t rows, int64_t cols, float maxq, float* scale,
                    float* zero, hipStream_t s);

// ------------------------------------------------------------- objective
size_t objective_ws_bytes(int64_t d_out, int64_t d_in);
kq_status objective_run(const float* W0, const float* What, const float* HX, const float* D,
                        const float* HG, int64_t d_out, int64_t d_in, double* obj, Arena& ws,
                        hipStream_t s);

// -------------------------------------------------------------- inference
int64_t packed_row_words(int64_t d_in, int bits);
kq_status pack_run(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed,
                   hipStream_t s);
size_t apply_a4_ws_bytes(int64_t d_out, int64_t d_in, int64_t batch);
kq_status apply_a4_run(const uint32_t* packed, const float* scale, const float* zero,
                       const float* s_x, const float* s_g, const int8_t* si, const int8_t* so,
                       int64_t bi, int64_t bo, const float* x, int64_t batch, int64_t d_out,
                       int64_t d_in, float clip, float* y, int8_t* codes_out, float* scale_out,
                       Arena& ws, hipStream_t s);
size_t apply_ws_bytes(int64_t d_out, int64_t d_in, int64_t batch);
kq_status apply_run(const uint32_t* packed, int bits, const float* scale, const float* zero,
                    int group, const float* s_x, const float* s_g, const int8_t* si,
                    const int8_t* so, int64_t bi, int64_t bo, const float* x, int64_t batch,
                    int64_t d_out, int64_t d_in, float* y, Arena& ws, hipStream_t s);

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace kq
