// C ABI of libkq: argument validation on the host, workspace sizing, and the
// orchestration of each stage's kernels on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>
#include <algorithm>
#include <mutex>

#include "kq_internal.h"

namespace kq {

namespace {
thread_local char g_err[512] = "";
}

kq_status fail(kq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kq_status hip_fail(hipError_t e, const char* where) {
  snprintf(g_err, sizeof(g_err), "HIP error %d (%s) in %s", int(e), hipGetErrorString(e), where);
  return KQ_ERR_HIP;
}

void clear_error() { g_err[0] = 0; }

namespace {
// per op: events recorded around the op's main kernel
constexpr int N_OPS = 10;
thread_local hipEvent_t g_kernel_ev[N_OPS][2] = {};
}

kq_status mark_kernel(kq_op op, int edge, hipStream_t s) {
  if (op < 0 || op >= N_OPS || g_kernel_ev[op][edge] == nullptr) return KQ_OK;
  KQ_HIP(hipEventRecord(g_kernel_ev[op][edge], s));
  return KQ_OK;
}

namespace {
// Pinned host landing area for results read back to the host, one per
// thread, allocated on first use and kept until the process ends.
constexpr size_t READBACK_BYTES = 64;
thread_local void* g_readback = nullptr;
}

kq_status read_to_host(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes > READBACK_BYTES) return fail(KQ_ERR_ARG, "internal read-back of %zu bytes", bytes);
  if (!g_readback) KQ_HIP(hipHostMalloc(&g_readback, READBACK_BYTES, hipHostMallocDefault));
  // A copy into pinned memory is truly asynchronous, and polling the stream
  // notices its completion within microseconds; a blocking synchronize (and
  // a copy into pageable memory, which waits the same way) wakes the host
  // only about 0.1 ms after the device has gone idle.
  KQ_HIP(hipMemcpyAsync(g_readback, src, bytes, hipMemcpyDeviceToHost, s));
  hipError_t e;
  while ((e = hipStreamQuery(s)) == hipErrorNotReady) {
  }
  KQ_HIP(e);
  memcpy(dst, g_readback, bytes);
  return KQ_OK;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int64_t lowbit(int64_t v) { return v & (-v); }

kq_status check_ws(const void* ws, size_t have, size_t need, const char* who) {
  if (need == 0) return KQ_OK;
  if (!ws) return fail(KQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got NULL", who, need);
  if (have < need)
    return fail(KQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need, have);
  if (!aligned16(ws)) return fail(KQ_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  return KQ_OK;
}

kq_status resolve_block(int64_t d, int64_t blk, int64_t* out, const char* side) {
  int64_t b = blk == 0 ? lowbit(d) : blk;
  if (blk < 0 || !pow2(b) || d % b != 0)
    return fail(KQ_ERR_SHAPE, "biip: %s Hadamard block %lld must be a power of two dividing %lld", side,
                (long long)b, (long long)d);
  if (b > 8192)
    return fail(KQ_ERR_UNSUPPORTED, "biip: %s Hadamard block %lld exceeds 8192", side, (long long)b);
  *out = b;
  return KQ_OK;
}

kq_status check_cfg(const kq_quant_cfg* cfg, int64_t d_in) {
  if (!cfg) return fail(KQ_ERR_ARG, "gptaq_quantize: cfg is NULL");
  if (cfg->bits < 1 || cfg->bits > 8) return fail(KQ_ERR_ARG, "gptaq_quantize: bits must be in [1, 8]");
  if (cfg->group != 0 && cfg->group != 128)
    return fail(KQ_ERR_UNSUPPORTED, "gptaq_quantize: group must be 0 (per channel) or 128");
  if (cfg->block != 128) return fail(KQ_ERR_UNSUPPORTED, "gptaq_quantize: block must be 128");
  if (cfg->flags != 0) return fail(KQ_ERR_ARG, "gptaq_quantize: flags must be 0");
  if (d_in < 128 || d_in % 128 != 0)
    return fail(KQ_ERR_SHAPE, "gptaq_quantize: d_in must be a positive multiple of 128");
  return KQ_OK;
}

}  // namespace
}  // namespace kq

using namespace kq;

// Scratch memory of kq_apply_quantized_noalloc: one copy per device, held
// until the process ends. Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol); the device
// address of each GPU's copy comes from hipGetSymbolAddress, called once per
// device with that device current, and is kept in noalloc_ptr.
static __device__ __align__(256) unsigned char scratch[KQ_NOALLOC_SCRATCH_BYTES];

namespace {

// argument checks shared by kq_apply_quantized and its no-allocation variant
kq_status apply_validate(const uint32_t* packed, int32_t bits, const float* scale, const float* zero,
                         int32_t group, const float* s_x, const float* s_g, const int8_t* sign_in,
                         const int8_t* sign_out, int64_t blk_in, int64_t blk_out, const float* x,
                         int64_t batch, int64_t d_out, int64_t d_in, float* y, int64_t* bi,
                         int64_t* bo) {
  if (!packed || !scale || !zero || !s_x || !s_g || !sign_in || !sign_out || !x || !y)
    return fail(KQ_ERR_ARG, "apply_quantized: NULL argument");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(KQ_ERR_ARG, "apply_quantized: bits must be 2, 3, 4 or 8");
  if (group != 0 && group != 128)
    return fail(KQ_ERR_UNSUPPORTED, "apply_quantized: group must be 0 or 128");
  if (d_out < 4 || d_out % 4 || batch < 1 || batch > 65536)
    return fail(KQ_ERR_SHAPE, "apply_quantized: d_out must be a multiple of 4 and 1 <= batch <= 65536");
  if (d_in < 32 || d_in % 32 || (group && d_in % group))
    return fail(KQ_ERR_SHAPE, "apply_quantized: d_in must be a multiple of 32 (of the group size)");
  KQ_TRY(resolve_block(d_in, blk_in, bi, "input"));
  KQ_TRY(resolve_block(d_out, blk_out, bo, "output"));
  const void* ptrs[4] = {packed, x, y, s_x};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(KQ_ERR_ARG, "apply_quantized: packed, x, y, s_x must be 16-byte aligned");
  return KQ_OK;
}

constexpr int MAX_DEVICES = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[MAX_DEVICES] = {};

kq_status noalloc_scratch(void** out) {
  int dev = -1;
  KQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(KQ_ERR_UNSUPPORTED, "apply_quantized_noalloc: device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* p = nullptr;
    KQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(KQ_ERR_HIP, "apply_quantized_noalloc: no device address for the scratch array");
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return KQ_OK;
}

}  // namespace

extern "C" {

const char* kq_last_error(void) { return g_err; }

const char* kq_version(void) { return "kq 0.1 gfx950"; }

kq_status kq_set_gemm_tile(int tile) {
  clear_error();
  if (tile != 0 && tile != 3 && tile != 64 && tile != 128 && tile != 256)
    return fail(KQ_ERR_ARG, "set_gemm_tile: tile must be 0 (by shape), 3 (three bf16 terms), 64, 128 or 256");
  set_gemm_tile(tile);
  return KQ_OK;
}

kq_status kq_set_kernel_events(kq_op op, hipEvent_t start, hipEvent_t stop) {
  clear_error();
  if (op != KQ_OP_ACCUMULATE_COV && op != KQ_OP_GPTAQ_QUANTIZE && op != KQ_OP_APPLY_QUANTIZED &&
      op != KQ_OP_APPLY_QUANTIZED_A4)
    return fail(KQ_ERR_UNSUPPORTED,
                "set_kernel_events: only KQ_OP_ACCUMULATE_COV, KQ_OP_GPTAQ_QUANTIZE and the two "
                "KQ_OP_APPLY_QUANTIZED ops have a timed kernel");
  if ((start == nullptr) != (stop == nullptr))
    return fail(KQ_ERR_ARG, "set_kernel_events: pass both events or neither");
  g_kernel_ev[op][0] = start;
  g_kernel_ev[op][1] = stop;
  return KQ_OK;
}

kq_status kq_workspace_size(kq_op op, int64_t d_out, int64_t d_in, int64_t n_tok, kq_dtype dtype,
                            const kq_quant_cfg* cfg, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(KQ_ERR_ARG, "workspace_size: bytes is NULL");
  *bytes = 0;
  if (d_in < 1) return fail(KQ_ERR_SHAPE, "workspace_size: d_in must be >= 1");
  switch (op) {
    case KQ_OP_ACCUMULATE_COV:
      if (d_out < 1 || n_tok < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      if (dtype != KQ_BF16 && dtype != KQ_F32) return fail(KQ_ERR_ARG, "workspace_size: bad dtype");
      // the largest need over every subset of outputs a call may request
      for (int m = 1; m < 8; ++m)
        *bytes = std::max(*bytes, cov_ws_bytes(n_tok, d_in, d_out, dtype, m & 1, m & 2, m & 4));
      return KQ_OK;
    case KQ_OP_BIIP:
      if (d_out < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      *bytes = biip_ws_bytes(d_out, d_in);
      return KQ_OK;
    case KQ_OP_SENSITIVITY: {
      Arena ar{nullptr, 0, 0};
      ar.take<double>(2);
      *bytes = ar.used;
      return KQ_OK;
    }
    case KQ_OP_CHOLESKY_INV:
      *bytes = chol_ws_bytes(d_in);
      return KQ_OK;
    case KQ_OP_FORM_P: {
      Arena ar{nullptr, 0, 0};
      ar.take<float>(size_t(d_in) * d_in);
      *bytes = ar.used;
      return KQ_OK;
    }
    case KQ_OP_GPTAQ_QUANTIZE:
      if (d_out < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      *bytes = gptaq_ws_bytes(d_out, d_in, cfg ? cfg->group : 0, true);
      return KQ_OK;
    case KQ_OP_LAYER_OBJECTIVE:
      if (d_out < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      *bytes = objective_ws_bytes(d_out, d_in);
      return KQ_OK;
    case KQ_OP_APPLY_QUANTIZED:
      if (d_out < 1 || n_tok < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      *bytes = apply_ws_bytes(d_out, d_in, n_tok);
      return KQ_OK;
    case KQ_OP_YAQA_QUANTIZE:
      if (d_out < 1 || d_in < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      *bytes = yaqa_ws_bytes(d_out, d_in, true);
      return KQ_OK;
    case KQ_OP_APPLY_QUANTIZED_A4:
      if (d_out < 1 || n_tok < 1) return fail(KQ_ERR_SHAPE, "workspace_size: bad sizes");
      *bytes = apply_a4_ws_bytes(d_out, d_in, n_tok);
      return KQ_OK;
  }
  return fail(KQ_ERR_ARG, "workspace_size: unknown op %d", int(op));
}

kq_status kq_accumulate_cov(const void* X, const void* Xq, const void* G, kq_dtype dt, int64_t n_tok,
                            int64_t d_in, int64_t d_out, float alpha, float beta, float* HX, float* D,
                            float* HG, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (dt != KQ_BF16 && dt != KQ_F32) return fail(KQ_ERR_ARG, "accumulate_cov: bad dtype %d", int(dt));
  if (!HX && !D && !HG) return fail(KQ_ERR_ARG, "accumulate_cov: no output requested");
  if ((HX || D) && !Xq) return fail(KQ_ERR_ARG, "accumulate_cov: HX and D need Xq");
  if (D && !X) return fail(KQ_ERR_ARG, "accumulate_cov: D needs X");
  if (HG && !G) return fail(KQ_ERR_ARG, "accumulate_cov: HG needs G");
  if (n_tok < 1 || ((HX || D) && d_in < 1) || (HG && d_out < 1))
    return fail(KQ_ERR_SHAPE, "accumulate_cov: sizes must be >= 1");
  if (((HX || D) && d_in % 8) || (HG && d_out % 8))
    return fail(KQ_ERR_SHAPE, "accumulate_cov: d_in and d_out must be multiples of 8");
  if (dt == KQ_F32 && n_tok % 4)
    return fail(KQ_ERR_SHAPE, "accumulate_cov: fp32 inputs need n_tok to be a multiple of 4");
  if (!std::isfinite(alpha) || !std::isfinite(beta))
    return fail(KQ_ERR_ARG, "accumulate_cov: alpha and beta must be finite");
  const void* ptrs[6] = {X, Xq, G, HX, D, HG};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(KQ_ERR_ARG, "accumulate_cov: buffers must be 16-byte aligned");
  const size_t need = cov_ws_bytes(n_tok, d_in, d_out, dt, HX != nullptr, D != nullptr, HG != nullptr);
  KQ_TRY(check_ws(ws, ws_bytes, need, "accumulate_cov"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return cov_run(X, Xq, G, dt, n_tok, d_in, d_out, alpha, beta, HX, D, HG, ar, stream);
}

kq_status kq_biip(float* W, float* HX, float* D, float* HG, int64_t d_out, int64_t d_in,
                  const int8_t* sign_in, const int8_t* sign_out, int64_t blk_in, int64_t blk_out,
                  float* s_x, float* s_g, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!W || !HX || !HG || !sign_in || !sign_out) return fail(KQ_ERR_ARG, "biip: NULL argument");
  if (d_out < 4 || d_in < 4 || d_out % 4 || d_in % 4)
    return fail(KQ_ERR_SHAPE, "biip: d_out and d_in must be multiples of 4");
  const void* ptrs[4] = {W, HX, D, HG};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(KQ_ERR_ARG, "biip: buffers must be 16-byte aligned");
  int64_t bi = 0, bo = 0;
  KQ_TRY(resolve_block(d_in, blk_in, &bi, "input"));
  KQ_TRY(resolve_block(d_out, blk_out, &bo, "output"));
  KQ_TRY(check_ws(ws, ws_bytes, biip_ws_bytes(d_out, d_in), "biip"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return biip_run(W, HX, D, HG, d_out, d_in, sign_in, sign_out, bi, bo, s_x, s_g, ar, stream);
}

kq_status kq_sensitivity(const float* HX, const float* HG, int64_t d_in, int64_t d_out, double* trHX,
                         double* trHG, double* s, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!HX || !HG) return fail(KQ_ERR_ARG, "sensitivity: NULL argument");
  if (d_in < 1 || d_out < 1) return fail(KQ_ERR_SHAPE, "sensitivity: sizes must be >= 1");
  Arena sz{nullptr, 0, 0};
  sz.take<double>(2);
  KQ_TRY(check_ws(ws, ws_bytes, sz.used, "sensitivity"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  double* dev = ar.take<double>(2);
  KQ_TRY(diag_sum(HX, d_in, dev, stream));
  KQ_TRY(diag_sum(HG, d_out, dev + 1, stream));
  double h[2] = {0.0, 0.0};
  KQ_TRY(read_to_host(h, dev, sizeof(h), stream));
  if (trHX) *trHX = h[0];
  if (trHG) *trHG = h[1];
  if (s) *s = h[0] * h[1];
  if (!std::isfinite(h[0]) || !std::isfinite(h[1]))
    return fail(KQ_ERR_NONFINITE, "sensitivity: non-finite trace");
  return KQ_OK;
}

kq_status kq_cholesky_inv(const float* H, int64_t n, float damp, float* U, int32_t* info, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (info) *info = 0;
  if (!H || !U) return fail(KQ_ERR_ARG, "cholesky_inv: NULL argument");
  if (H == U) return fail(KQ_ERR_ARG, "cholesky_inv: H and U must be distinct buffers");
  if (n < 128 || n % 128) return fail(KQ_ERR_SHAPE, "cholesky_inv: n must be a positive multiple of 128");
  if (!std::isfinite(damp) || damp < 0.f) return fail(KQ_ERR_ARG, "cholesky_inv: damp must be finite and >= 0");
  if (!aligned16(H) || !aligned16(U)) return fail(KQ_ERR_ARG, "cholesky_inv: buffers must be 16-byte aligned");
  KQ_TRY(check_ws(ws, ws_bytes, chol_ws_bytes(n), "cholesky_inv"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return chol_inv_run(H, n, damp, U, info, ar, stream);
}

kq_status kq_form_p(const float* D, const float* U, int64_t n, float* P, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  clear_error();
  if (!D || !U || !P) return fail(KQ_ERR_ARG, "form_p: NULL argument");
  if (P == D || P == U) return fail(KQ_ERR_ARG, "form_p: P must not alias D or U");
  if (n < 128 || n % 128) return fail(KQ_ERR_SHAPE, "form_p: n must be a positive multiple of 128");
  if (!aligned16(D) || !aligned16(U) || !aligned16(P)) return fail(KQ_ERR_ARG, "form_p: buffers must be 16-byte aligned");
  Arena sz{nullptr, 0, 0};
  sz.take<float>(size_t(n) * n);
  KQ_TRY(check_ws(ws, ws_bytes, sz.used, "form_p"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return formp_run(D, U, n, P, ar, stream);
}

kq_status kq_gptaq_quantize(float* W, const float* U, const float* D, int64_t d_out, int64_t d_in,
                            const kq_quant_cfg* cfg, uint8_t* codes, float* scale, float* zero,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!W || !U || !codes || !scale || !zero) return fail(KQ_ERR_ARG, "gptaq_quantize: NULL argument");
  if (d_out < 1) return fail(KQ_ERR_SHAPE, "gptaq_quantize: d_out must be >= 1");
  KQ_TRY(check_cfg(cfg, d_in));
  const void* ptrs[3] = {W, U, D};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(KQ_ERR_ARG, "gptaq_quantize: buffers must be 16-byte aligned");
  KQ_TRY(check_ws(ws, ws_bytes, gptaq_ws_bytes(d_out, d_in, cfg->group, D != nullptr), "gptaq_quantize"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return gptaq_run(W, U, D, d_out, d_in, cfg->bits, cfg->group, codes, scale, zero, ar, stream);
}

kq_status kq_yaqa_quantize(float* W, const float* U_in, const float* U_out, const float* D,
                           int64_t d_out, int64_t d_in, const kq_quant_cfg* cfg, uint8_t* codes,
                           float* scale, float* zero, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  clear_error();
  if (!W || !U_in || !U_out || !codes || !scale || !zero)
    return fail(KQ_ERR_ARG, "yaqa_quantize: NULL argument");
  if (d_out < 1 || d_in < 1) return fail(KQ_ERR_SHAPE, "yaqa_quantize: d_out and d_in must be >= 1");
  if (!cfg) return fail(KQ_ERR_ARG, "yaqa_quantize: cfg is NULL");
  if (cfg->bits < 1 || cfg->bits > 8) return fail(KQ_ERR_ARG, "yaqa_quantize: bits must be in [1, 8]");
  if (cfg->group != 0)
    return fail(KQ_ERR_UNSUPPORTED, "yaqa_quantize: group must be 0 (one grid per output channel)");
  if (cfg->block != 128) return fail(KQ_ERR_UNSUPPORTED, "yaqa_quantize: block must be 128");
  if (cfg->flags != 0) return fail(KQ_ERR_ARG, "yaqa_quantize: flags must be 0");
  if (d_out > (int64_t(1) << 24) || d_in > (int64_t(1) << 24))
    return fail(KQ_ERR_SHAPE, "yaqa_quantize: dimensions above 2^24 are not supported");
  const void* ptrs[4] = {W, U_in, U_out, D};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(KQ_ERR_ARG, "yaqa_quantize: buffers must be 16-byte aligned");
  KQ_TRY(check_ws(ws, ws_bytes, yaqa_ws_bytes(d_out, d_in, D != nullptr), "yaqa_quantize"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return yaqa_run(W, U_in, U_out, D, d_out, d_in, cfg->bits, codes, scale, zero, ar, stream);
}

kq_status kq_allocate_bits(const double* s, const int64_t* n_params, int32_t L, const int32_t* widths,
                           int32_t n_widths, double avg_budget, int32_t* bits_out) {
  clear_error();
  if (!s || !n_params || !widths || !bits_out) return fail(KQ_ERR_ARG, "allocate_bits: NULL argument");
  if (L < 1 || n_widths < 1) return fail(KQ_ERR_ARG, "allocate_bits: L and n_widths must be >= 1");
  if (!std::isfinite(avg_budget)) return fail(KQ_ERR_ARG, "allocate_bits: budget must be finite");
  std::vector<int32_t> ws(widths, widths + n_widths);
  std::sort(ws.begin(), ws.end());
  for (int32_t k = 0; k < n_widths; ++k)
    if (ws[k] < 1 || (k && ws[k] == ws[k - 1])) return fail(KQ_ERR_ARG, "allocate_bits: widths must be distinct and >= 1");
  double total = 0.0;
  for (int32_t l = 0; l < L; ++l) {
    if (n_params[l] < 0) return fail(KQ_ERR_ARG, "allocate_bits: negative parameter count");
    if (!std::isfinite(s[l])) return fail(KQ_ERR_NONFINITE, "allocate_bits: non-finite sensitivity");
    total += double(n_params[l]);
  }
  const int32_t wmin = ws.front();
  const double budget = avg_budget * total;
  double used = double(wmin) * total;
  if (used > budget) return fail(KQ_ERR_ARG, "allocate_bits: budget is below the narrowest width");
  std::vector<int32_t> order(L);
  for (int32_t l = 0; l < L; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return s[a] > s[b]; });
  for (int32_t l = 0; l < L; ++l) bits_out[l] = wmin;
  for (int32_t idx : order) {
    for (int32_t k = n_widths - 1; k >= 0; --k) {
      const double extra = double(ws[k] - wmin) * double(n_params[idx]);
      if (used + extra <= budget) {
        bits_out[idx] = ws[k];
        used += extra;
        break;
      }
    }
  }
  return KQ_OK;
}

kq_status kq_layer_objective(const float* W0, const float* What, const float* HX, const float* D,
                             const float* HG, int64_t d_out, int64_t d_in, double* obj, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!W0 || !What || !HX || !HG || !obj) return fail(KQ_ERR_ARG, "layer_objective: NULL argument");
  if (d_out < 4 || d_in < 4 || d_out % 4 || d_in % 4)
    return fail(KQ_ERR_SHAPE, "layer_objective: d_out and d_in must be multiples of 4");
  const void* ptrs[5] = {W0, What, HX, D, HG};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(KQ_ERR_ARG, "layer_objective: buffers must be 16-byte aligned");
  KQ_TRY(check_ws(ws, ws_bytes, objective_ws_bytes(d_out, d_in), "layer_objective"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return objective_run(W0, What, HX, D, HG, d_out, d_in, obj, ar, stream);
}

kq_status kq_packed_row_words(int64_t d_in, int32_t bits, int64_t* words) {
  clear_error();
  if (!words) return fail(KQ_ERR_ARG, "packed_row_words: words is NULL");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(KQ_ERR_ARG, "packed_row_words: bits must be 2, 3, 4 or 8");
  if (d_in < 1) return fail(KQ_ERR_SHAPE, "packed_row_words: d_in must be >= 1");
  *words = packed_row_words(d_in, bits);
  return KQ_OK;
}

kq_status kq_pack_codes(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits,
                        uint32_t* packed, hipStream_t stream) {
  clear_error();
  if (!codes || !packed) return fail(KQ_ERR_ARG, "pack_codes: NULL argument");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(KQ_ERR_ARG, "pack_codes: bits must be 2, 3, 4 or 8");
  if (d_out < 1 || d_in < 1) return fail(KQ_ERR_SHAPE, "pack_codes: bad sizes");
  if (!aligned16(packed)) return fail(KQ_ERR_ARG, "pack_codes: packed must be 16-byte aligned");
  return pack_run(codes, d_out, d_in, bits, packed, stream);
}

kq_status kq_apply_quantized(const uint32_t* packed, int32_t bits, const float* scale,
                             const float* zero, int32_t group, const float* s_x, const float* s_g,
                             const int8_t* sign_in, const int8_t* sign_out, int64_t blk_in,
                             int64_t blk_out, const float* x, int64_t batch, int64_t d_out,
                             int64_t d_in, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int64_t bi = 0, bo = 0;
  KQ_TRY(apply_validate(packed, bits, scale, zero, group, s_x, s_g, sign_in, sign_out, blk_in, blk_out,
                        x, batch, d_out, d_in, y, &bi, &bo));
  KQ_TRY(check_ws(ws, ws_bytes, apply_ws_bytes(d_out, d_in, batch), "apply_quantized"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return apply_run(packed, bits, scale, zero, group, s_x, s_g, sign_in, sign_out, bi, bo, x, batch,
                   d_out, d_in, y, ar, stream);
}

kq_status kq_apply_quantized_noalloc(const uint32_t* packed, int32_t bits, const float* scale,
                                     const float* zero, int32_t group, const float* s_x,
                                     const float* s_g, const int8_t* sign_in, const int8_t* sign_out,
                                     int64_t blk_in, int64_t blk_out, const float* x, int64_t batch,
                                     int64_t d_out, int64_t d_in, float* y, hipStream_t stream) {
  clear_error();
  int64_t bi = 0, bo = 0;
  KQ_TRY(apply_validate(packed, bits, scale, zero, group, s_x, s_g, sign_in, sign_out, blk_in, blk_out,
                        x, batch, d_out, d_in, y, &bi, &bo));
  const size_t need = apply_ws_bytes(d_out, d_in, batch);
  if (need > size_t(KQ_NOALLOC_SCRATCH_BYTES))
    return fail(KQ_ERR_WORKSPACE,
                "apply_quantized_noalloc: these sizes need %zu bytes of scratch, above the fixed %zu",
                need, size_t(KQ_NOALLOC_SCRATCH_BYTES));
  void* p = nullptr;
  KQ_TRY(noalloc_scratch(&p));
  Arena ar{static_cast<char*>(p), size_t(KQ_NOALLOC_SCRATCH_BYTES), 0};
  return apply_run(packed, bits, scale, zero, group, s_x, s_g, sign_in, sign_out, bi, bo, x, batch,
                   d_out, d_in, y, ar, stream);
}

kq_status kq_apply_quantized_a4(const uint32_t* packed, const float* scale, const float* zero,
                                const float* s_x, const float* s_g, const int8_t* sign_in,
                                const int8_t* sign_out, int64_t blk_in, int64_t blk_out,
                                const float* x, int64_t batch, int64_t d_out, int64_t d_in,
                                float clip, float* y, int8_t* act_codes, float* act_scale,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!packed || !scale || !zero || !s_x || !s_g || !sign_in || !sign_out || !x || !y)
    return fail(KQ_ERR_ARG, "apply_quantized_a4: NULL argument");
  if (!(clip > 0.f && clip <= 1.f))
    return fail(KQ_ERR_ARG, "apply_quantized_a4: clip must be in (0, 1]");
  if (d_out < 4 || d_out % 4 || batch < 1 || batch > 65536)
    return fail(KQ_ERR_SHAPE, "apply_quantized_a4: d_out must be a multiple of 4 and 1 <= batch <= 65536");
  if (d_in < 512 || d_in % 512)
    return fail(KQ_ERR_SHAPE, "apply_quantized_a4: d_in must be a multiple of 512");
  if (d_in > (int64_t(1) << 24))
    return fail(KQ_ERR_SHAPE, "apply_quantized_a4: d_in above 2^24");
  int64_t bi = 0, bo = 0;
  KQ_TRY(resolve_block(d_in, blk_in, &bi, "input"));
  KQ_TRY(resolve_block(d_out, blk_out, &bo, "output"));
  const void* ptrs[5] = {packed, x, y, s_x, act_codes};
  for (const void* p : ptrs)
    if (!aligned16(p))
      return fail(KQ_ERR_ARG, "apply_quantized_a4: packed, x, y, s_x, act_codes must be 16-byte aligned");
  KQ_TRY(check_ws(ws, ws_bytes, apply_a4_ws_bytes(d_out, d_in, batch), "apply_quantized_a4"));
  Arena ar{static_cast<char*>(ws), ws_bytes, 0};
  return apply_a4_run(packed, scale, zero, s_x, s_g, sign_in, sign_out, bi, bo, x, batch, d_out, d_in,
                      clip, y, act_codes, act_scale, ar, stream);
}

}  // extern "C"
