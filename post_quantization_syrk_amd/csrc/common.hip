// Error reporting, version and small utility kernels.
#include "kq_internal.h"

#include <string.h>

#include <atomic>

namespace kq {

static thread_local char g_last_error[512] = "";

kq_status fail(kq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

int device_cu_count() {
  // per device; threads that race to fill an entry store the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

constexpr int N_TESTING_KNOBS = 3;
static std::atomic<int64_t> g_testing[N_TESTING_KNOBS] = {{-1}, {-1}, {-1}};

int64_t testing_value(int knob, int64_t dflt) {
  if (knob < 0 || knob >= N_TESTING_KNOBS) return dflt;
  const int64_t v = g_testing[knob].load(std::memory_order_relaxed);
  return v < 0 ? dflt : v;
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

kq_status fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return KQ_OK;
  int64_t blocks = ceil_div(n, 256);
  if (blocks > 8192) blocks = 8192;
  fill_f32_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n, v);
  KQ_LAUNCHED("fill_f32_kernel");
  return KQ_OK;
}

kq_status fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return KQ_OK;
  int64_t blocks = ceil_div(n, 256);
  if (blocks > 8192) blocks = 8192;
  fill_u32_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n, v);
  KQ_LAUNCHED("fill_u32_kernel");
  return KQ_OK;
}

}  // namespace kq

extern "C" int kq_version(void) { return 200; /* 0.2.0: act_order, w_clip */ }

extern "C" const char* kq_last_error(void) { return kq::g_last_error; }

extern "C" kq_status kq_testing_select(int knob, int64_t value) {
  if (knob < 0 || knob >= kq::N_TESTING_KNOBS)
    return kq::fail(KQ_EINVAL, "kq_testing_select: unknown knob %d", knob);
  if (value < -1) return kq::fail(KQ_EINVAL, "kq_testing_select: value %lld", (long long)value);
  kq::g_testing[knob].store(value, std::memory_order_relaxed);
  return KQ_OK;
}
