/*
 * kq_testing.h -- path selection for the engine's own tests (C ABI of libkq.so).
 *
 * Some operations have more than one implementation that computes the same result (a
 * fallback kernel for inputs the default one cannot take, or a restructured schedule that
 * performs the same arithmetic).  The library picks among them by shape; a test can force
 * one, to check that every path agrees with the oracle or, bit for bit, with the default.
 * Production callers never need this: with nothing selected every path is the default.
 * The selection is process-wide and applies to calls made after it returns.
 */
#ifndef KQ_TESTING_H
#define KQ_TESTING_H

#include <stdint.h>

#include "kq.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  /* kq_accumulate_hessian's kernel: 4 = direct-to-LDS (the default), 0 .. 3 = the
   * register-staged kernel that serves strides too large for the default (bit 0: 8 waves
   * instead of 4; bit 1: split-major workgroup order). */
  KQ_TESTING_SYRK_KERNEL = 0,
  /* Columns per super-block of kq_quantize_layer's factorization (a multiple of 128;
   * default 1024 for factors larger than 128 MB, else the whole width): each block's update
   * of the columns left of its super-block waits for one rank-(super-block) update.  The
   * same updates, summed in another order. */
  KQ_TESTING_FACTOR_SUPERBLOCK = 1,
  /* Longest row (bytes) the quantizer's row kernels stage in LDS (default 65536); 0 forces
   * their direct paths, which longer rows take. */
  KQ_TESTING_ROW_LDS_BYTES = 2
};

/* Selects `value` for `knob`; value -1 restores the default.  KQ_EINVAL for an unknown knob
 * or a value below -1.  Not thread-safe against concurrent engine calls. */
kq_status kq_testing_select(int knob, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* KQ_TESTING_H */
