// Trace reductions and the per-sublayer sensitivity tr(H_G) * tr(H_X).
//
// KronQ README, opening section: inter-layer mixed precision is guided by the
// tr(H_G) tr(H_X) sensitivity; KronQ arXiv abstract, point 2: the metric is
// driven by the gradient and activation Hessian traces.
#include "kq_internal.h"

#include <mutex>

namespace kq {
namespace {

// Per-device result slots of the two traces (each device holds its own copy).
__device__ double g_trace_out[2];

std::mutex g_trace_mutex;

// One block per matrix: fp64 sum of the fp32 diagonal, fixed reduction order.
__global__ __launch_bounds__(256) void trace2_kernel(const float* __restrict__ HX, int64_t nx,
                                                     int64_t ldx, const float* __restrict__ HG,
                                                     int64_t ng, int64_t ldg, double* out) {
  const float* H = blockIdx.x == 0 ? HX : HG;
  const int64_t n = blockIdx.x == 0 ? nx : ng;
  const int64_t ld = blockIdx.x == 0 ? ldx : ldg;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += (double)H[i * ld + i];
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_sensitivity(const float* HX, int64_t n_in, int64_t ldx, const float* HG,
                                    int64_t n_out, int64_t ldg, double out3[3], void* stream) {
  using namespace kq;
  if (!HX || !HG || !out3) return fail(KQ_EINVAL, "kq_sensitivity: NULL argument");
  if (n_in < 1 || n_out < 1 || ldx < n_in || ldg < n_out)
    return fail(KQ_ESHAPE, "kq_sensitivity: bad sizes");
  hipStream_t s = as_stream(stream);
  std::lock_guard<std::mutex> lock(g_trace_mutex);
  double* dev = nullptr;
  KQ_HIP(hipGetSymbolAddress((void**)&dev, HIP_SYMBOL(g_trace_out)));
  trace2_kernel<<<dim3(2), dim3(256), 0, s>>>(HX, n_in, ldx, HG, n_out, ldg, dev);
  KQ_LAUNCHED("trace2_kernel");
  double host[2];
  KQ_HIP(hipMemcpyAsync(host, dev, sizeof(host), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  out3[0] = host[0];
  out3[1] = host[1];
  out3[2] = host[1] * host[0];
  return KQ_OK;
}
