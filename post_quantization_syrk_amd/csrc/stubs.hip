// Entry points whose kernels are not in this build yet.
#include "kq_internal.h"

extern "C" kq_status kq_biip_rotate(const float*, float*, int64_t, int64_t, const float*, float*,
                                    const float*, float*, const int8_t*, const int8_t*, int64_t,
                                    int64_t, float, int, float*, float*, void*) {
  return kq::fail(KQ_ENOTIMPL, "kq_biip_rotate: not implemented");
}

extern "C" kq_status kq_quantize_layer_workspace(const kq_quant_params*, int64_t, int64_t, int,
                                                 size_t* bytes) {
  if (bytes) *bytes = 0;
  return kq::fail(KQ_ENOTIMPL, "kq_quantize_layer_workspace: not implemented");
}

extern "C" kq_status kq_quantize_layer(const kq_quant_params*, float*, const float*, const float*,
                                       int64_t, int64_t, uint32_t*, float*, uint8_t*, uint8_t*,
                                       double*, void*, size_t, void*) {
  return kq::fail(KQ_ENOTIMPL, "kq_quantize_layer: not implemented");
}
