// Inter-layer bit allocation from tr(H_G) * tr(H_X) sensitivities (host code).
//
// KronQ README, opening section (the bit width of each sublayer is set from the
// product of its two factors' traces) and flags table
// (--inter_layer_mp); KronQ arXiv abstract, point 2.  The pages do not give
// the rule.  This engine's rule: a sublayer's expected loss behaves like
// s_l * 4^-b_l (uniform quantization noise of variance ~ 4^-b gives
// E tr(H_G dW H_X dW^T) ~ 4^-b tr(H_G) tr(H_X)).  Starting from the smallest
// width, the sublayer with the largest loss reduction per added bit-weight
// moves up one allowed width while the integer budget allows; ties go to the
// smallest index.  Compiled without floating-point contraction so every gain
// is the same two IEEE roundings (multiply, then divide) on any host.
#include "kq_internal.h"

#include <math.h>

#include <algorithm>
#include <vector>

extern "C" kq_status kq_allocate_bits(const double* sens, const int64_t* numel, int64_t L,
                                      const int* allowed, int n_allowed, int64_t target_num,
                                      int64_t target_den, int* bits_out) {
  using kq::fail;
  if (L < 0 || L > (int64_t)1 << 24) return fail(KQ_ESHAPE, "kq_allocate_bits: bad L");
  if (L == 0) return KQ_OK;
  if (!sens || !numel || !allowed || !bits_out)
    return fail(KQ_EINVAL, "kq_allocate_bits: NULL argument");
  if (n_allowed < 1 || n_allowed > 16) return fail(KQ_EINVAL, "kq_allocate_bits: n_allowed");
  if (target_num <= 0 || target_den <= 0)
    return fail(KQ_EINVAL, "kq_allocate_bits: target must be positive");
  std::vector<int> widths(allowed, allowed + n_allowed);
  std::sort(widths.begin(), widths.end());
  for (int i = 0; i < n_allowed; ++i) {
    if (widths[i] < 1 || widths[i] > 16) return fail(KQ_EINVAL, "kq_allocate_bits: width range");
    if (i && widths[i] == widths[i - 1]) return fail(KQ_EINVAL, "kq_allocate_bits: duplicates");
  }
  __int128 total = 0;
  for (int64_t l = 0; l < L; ++l) {
    if (numel[l] <= 0 || numel[l] > ((int64_t)1 << 40))
      return fail(KQ_EINVAL, "kq_allocate_bits: numel[%lld] out of range", (long long)l);
    if (!(sens[l] >= 0.0) || !isfinite(sens[l]))
      return fail(KQ_EINVAL, "kq_allocate_bits: sens[%lld] must be finite and >= 0", (long long)l);
    total += numel[l];
  }
  const __int128 budget = total * target_num / target_den;
  __int128 used = total * widths[0];
  std::vector<int> level(L, 0);
  for (;;) {
    int64_t best = -1;
    double best_gain = -1.0;
    for (int64_t l = 0; l < L; ++l) {
      const int i = level[l];
      if (i + 1 >= n_allowed) continue;
      const int b = widths[i], nb = widths[i + 1];
      if (used + (__int128)(nb - b) * numel[l] > budget) continue;
      const double dq = ldexp(1.0, -2 * b) - ldexp(1.0, -2 * nb);
      const double gain = (sens[l] * dq) / (double)(numel[l] * (int64_t)(nb - b));
      if (gain > best_gain) {
        best = l;
        best_gain = gain;
      }
    }
    if (best < 0) break;
    const int i = level[best];
    used += (__int128)(widths[i + 1] - widths[i]) * numel[best];
    level[best] = i + 1;
  }
  for (int64_t l = 0; l < L; ++l) bits_out[l] = widths[level[l]];
  return KQ_OK;
}
