// Internal helpers shared by the engine's HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/kq.h"
#include "../../include/kq_testing.h"

namespace kq {

// Records a thread-local message and returns `s`.
kq_status fail(kq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// The value a test selected for `knob` with kq_testing_select, or `dflt` when none is set.
int64_t testing_value(int knob, int64_t dflt);

// fp32 fill kernel launcher (used instead of hipMemsetAsync so captured graphs stay valid).
kq_status fill_f32(float* p, int64_t n, float v, hipStream_t s);
kq_status fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

// fp32 matrix operations used by the quantizer (gemm_f32.hip).
// C[M x N] (+)= alpha * op(A) op(B); row-major, op = transpose when the flag is set.
// Only tiles with tile_row <= tile_col are computed when upper_only is set.
// split_k > 1 adds partial products with atomics (C must be pre-initialized).
struct GemmArgs {
  int64_t M, N, K;
  const float* A; int64_t lda; bool transA;
  const float* B; int64_t ldb; bool transB;
  float* C; int64_t ldc;
  float alpha;        // scale of the product
  bool accumulate;    // C += alpha*AB (else C = alpha*AB)
  bool upper_only;    // only tiles with row-tile <= col-tile
  bool a_upper;       // op(A) is upper triangular (zeros below): skip K below the tile's rows
  bool b_upper;       // op(B) is upper triangular: skip K beyond the tile's columns
  int split_k;        // >= 1; > 1 requires accumulate (atomics) or partial_stride
  int batch;          // >= 1 independent products, operands offset by the strides below
  int64_t strideA, strideB, strideC;  // in elements
  // reduce epilogue: instead of writing C, accumulate sum(alpha*AB .* D) into *red (fp64)
  const float* D; int64_t ldd; double* red;
  // split partials: with partial_stride > 0, split z of the K range stores alpha times its
  // partial product to C + z * partial_stride (plain stores; C is not read).  The number of
  // splits launched (none of them empty) goes to *splits_used when that is not NULL.
  int64_t partial_stride;
  int* splits_used;
};
kq_status gemm_f32(const GemmArgs& g, hipStream_t s);

// U = R^-1 (explicit upper triangular, k x k, ld k; k % 128 == 0) for M + lambda I = R R^T,
// lambda = damp * mean(diag M); zero diagonals count as 1 and are flagged in dead (k bytes).
// F: k * k and Tsc: 128 * k floats of scratch; lam: 1 double; flag: set on a non-positive
// pivot (flipflop.hip).
kq_status explicit_inverse_factor(const float* M, int64_t k, float damp, float* F, float* Tsc,
                                  uint8_t* dead, double* lam, int* flag, float* U, hipStream_t s);

// H's lower block triangle (+)= sum_t A[t, i] B[t, j] over T tokens of two bf16 streams of n
// channels (16-byte aligned, strides multiples of 8), then optionally the lower triangle
// mirrored into the upper one; B == A forms the Hessian A^T A (syrk.hip).
kq_status gram_lower(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t T,
                     int64_t n, float* H, int64_t ldh, bool accumulate, bool mirror, hipStream_t s);

}  // namespace kq

#define KQ_HIP(expr)                                                                  \
  do {                                                                                \
    hipError_t _e = (expr);                                                           \
    if (_e != hipSuccess)                                                             \
      return ::kq::fail(KQ_EHIP, "%s failed: %s", #expr, hipGetErrorString(_e));      \
  } while (0)

#define KQ_LAUNCHED(name)                                                             \
  do {                                                                                \
    hipError_t _e = hipGetLastError();                                                \
    if (_e != hipSuccess)                                                             \
      return ::kq::fail(KQ_EHIP, "launch of %s failed: %s", name, hipGetErrorString(_e)); \
  } while (0)

#define KQ_TRY(expr)                   \
  do {                                 \
    kq_status _s = (expr);             \
    if (_s != KQ_OK) return _s;        \
  } while (0)
