// Trace reductions and the per-sublayer sensitivity tr(H_G) * tr(H_X).
//
// KronQ README, opening section: inter-layer mixed precision is guided by the
// tr(H_G) tr(H_X) sensitivity; KronQ arXiv abstract, point 2: the metric comes from
// the traces of the gradient and the activation factor.
#include "kq_internal.h"

#include <mutex>

namespace kq {
namespace {

// Per-device result slots of the traces and their product (each device holds its own copy).
__device__ double g_trace_out[3];

std::mutex g_trace_mutex;

// One workgroup: fp64 sums of the two fp32 diagonals (thread i adds entries i, i + 256, ..;
// then a fixed tree), out = {tr H_X, tr H_G, tr H_G * tr H_X}.
__device__ __forceinline__ double diag_sum(const float* __restrict__ H, int64_t n, int64_t ld,
                                           double* red) {
  // the same order as one entry at a time; eight loads in flight per thread (indices past n
  // read the last entry and count as zero, a select rather than a branch around the load)
  double s = 0.0;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += 8 * (int64_t)blockDim.x) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t i = min(i0 + (int64_t)k * blockDim.x, n - 1);
      v[k] = H[i * ld + i];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (i0 + (int64_t)k * blockDim.x < n) s += (double)v[k];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void trace2_kernel(const float* __restrict__ HX, int64_t nx,
                                                     int64_t ldx, const float* __restrict__ HG,
                                                     int64_t ng, int64_t ldg, double* out) {
  __shared__ double red[256];
  const double tx = diag_sum(HX, nx, ldx, red);
  const double tg = diag_sum(HG, ng, ldg, red);
  if (threadIdx.x == 0) {
    out[0] = tx;
    out[1] = tg;
    out[2] = tg * tx;
  }
}

kq_status check_sensitivity(const float* HX, int64_t n_in, int64_t ldx, const float* HG,
                            int64_t n_out, int64_t ldg, const void* out, const char* name) {
  if (!HX || !HG || !out) return fail(KQ_EINVAL, "%s: NULL argument", name);
  if (n_in < 1 || n_out < 1 || ldx < n_in || ldg < n_out)
    return fail(KQ_ESHAPE, "%s: bad sizes", name);
  return KQ_OK;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_sensitivity(const float* HX, int64_t n_in, int64_t ldx, const float* HG,
                                    int64_t n_out, int64_t ldg, double out3[3], void* stream) {
  using namespace kq;
  KQ_TRY(check_sensitivity(HX, n_in, ldx, HG, n_out, ldg, out3, "kq_sensitivity"));
  hipStream_t s = as_stream(stream);
  std::lock_guard<std::mutex> lock(g_trace_mutex);
  double* dev = nullptr;
  KQ_HIP(hipGetSymbolAddress((void**)&dev, HIP_SYMBOL(g_trace_out)));
  trace2_kernel<<<dim3(1), dim3(256), 0, s>>>(HX, n_in, ldx, HG, n_out, ldg, dev);
  KQ_LAUNCHED("trace2_kernel");
  double host[3];
  KQ_HIP(hipMemcpyAsync(host, dev, sizeof(host), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  out3[0] = host[0];
  out3[1] = host[1];
  out3[2] = host[2];
  return KQ_OK;
}

extern "C" kq_status kq_sensitivity_async(const float* HX, int64_t n_in, int64_t ldx,
                                          const float* HG, int64_t n_out, int64_t ldg,
                                          double* out3_dev, void* stream) {
  using namespace kq;
  KQ_TRY(check_sensitivity(HX, n_in, ldx, HG, n_out, ldg, out3_dev, "kq_sensitivity_async"));
  trace2_kernel<<<dim3(1), dim3(256), 0, as_stream(stream)>>>(HX, n_in, ldx, HG, n_out, ldg,
                                                               out3_dev);
  KQ_LAUNCHED("trace2_kernel");
  return KQ_OK;
}
