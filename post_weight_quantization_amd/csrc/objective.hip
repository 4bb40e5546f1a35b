// Layer objective (a metric, not a stage of the method).
//
// KronQ summary (hyper.ai), Method: the Kronecker-factored layer objective
// tr[H_G dW H_X dW^T] and its GPTAQ extension with the drift term, read as
//   obj = tr[H_G (dW H_X dW^T + 2 W0 D dW^T)],  dW = W0 - W^.
// Computed as M = dW H_X + 2 W0 D, K = M dW^T (fp32 MFMA GEMMs), then
// obj = sum_ik H_G[i][k] K[k][i] = <H_G, K>_F (H_G symmetric), summed in fp64.
#include "kq_internal.h"

namespace kq {

namespace {

__global__ void sub_kernel(const float* a, const float* b, float* c, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    c[i] = a[i] - b[i];
}

__global__ __launch_bounds__(256) void dot_partial_kernel(const float* a, const float* b, int64_t n,
                                                          double* part) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    acc += double(a[i]) * double(b[i]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void sum_kernel(const double* part, int n, double* out) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) acc += part[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

constexpr int NPART = 1024;

}  // namespace

size_t objective_ws_bytes(int64_t d_out, int64_t d_in) {
  Arena ar{nullptr, 0, 0};
  ar.take<float>(size_t(d_out) * d_in);   // dW
  ar.take<float>(size_t(d_out) * d_in);   // M
  ar.take<float>(size_t(d_out) * d_out);  // K
  ar.take<double>(NPART + 1);
  return ar.used;
}

kq_status objective_run(const float* W0, const float* What, const float* HX, const float* D,
                        const float* HG, int64_t d_out, int64_t d_in, double* obj, Arena& ws,
                        hipStream_t s) {
  float* dW = ws.take<float>(size_t(d_out) * d_in);
  float* M = ws.take<float>(size_t(d_out) * d_in);
  float* K = ws.take<float>(size_t(d_out) * d_out);
  double* part = ws.take<double>(NPART + 1);
  if (!dW || !M || !K || !part) return fail(KQ_ERR_WORKSPACE, "layer_objective: workspace too small");
  const int64_t nw = d_out * d_in;
  sub_kernel<<<unsigned(std::min<int64_t>(cdiv(nw, 256), 8192)), 256, 0, s>>>(W0, What, dW, nw);
  KQ_HIP(hipGetLastError());
  KQ_TRY(gemm_f32(gemm_args(dW, d_in, HX, d_in, M, d_in, d_out, d_in, d_in, 1.f, 0.f, 0), s));
  if (D) KQ_TRY(gemm_f32(gemm_args(W0, d_in, D, d_in, M, d_in, d_out, d_in, d_in, 2.f, 1.f, 0), s));
  KQ_TRY(gemm_f32(gemm_args(M, d_in, dW, d_in, K, d_out, d_out, d_out, d_in, 1.f, 0.f, G_TRANS_B), s));
  dot_partial_kernel<<<NPART, 256, 0, s>>>(HG, K, d_out * d_out, part);
  KQ_HIP(hipGetLastError());
  sum_kernel<<<1, 256, 0, s>>>(part, NPART, part + NPART);
  KQ_HIP(hipGetLastError());
  double h = 0.0;
  KQ_TRY(read_to_host(&h, part + NPART, sizeof(double), s));
  *obj = h;
  return KQ_OK;
}

}  // namespace kq
