// Damping and the reverse-order Cholesky factor of the processed H_X.
//
// GPTQ, which KronQ runs as its base quantizer (KronQ README, "Mapping paper
// results to flags": GPTQ is the baseline with no extra flags; the opening
// section: KronQ extends GPTQ/GPTAQ), rounds column by column through
// U = chol_upper(H_d^-1), H_d = H_X + lambda I, lambda = damp * mean(diag H_X).
// Here H_d = R R^T with R upper triangular is factored from the bottom-right
// corner up; then U = R^-1, since U^T U = R^-T R^-1 = H_d^-1 and U is upper
// with a positive diagonal (2 n^3 / 3 flops in all, against about 5 n^3 / 3
// for factor, invert, factor again).
//
// Reverse Cholesky, 64-column blocks from the last one up:
//   R22 R22^T = A22                  (one workgroup, in LDS)
//   R12 = A12 R22^-T                 (independent rows: one thread per row)
//   A11 -= R12 R12^T                 (fp32 MFMA, upper tiles only)
// Triangular inverse, 64-column blocks from the first one on:
//   U_JJ = R_JJ^-1                   (all diagonal blocks at once)
//   U_<J,J = -(U_<J,<J R_<J,J) U_JJ  (two fp32 MFMA products)
// The strictly lower triangle is cleared, so U is a plain upper-triangular matrix.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int NB = 64;
constexpr int LD = NB + 1;

// Dead channels (zero diagonal) get a unit diagonal; lambda = damp * mean(diag);
// lam_out[0] = lambda (fp64).  One workgroup.
__global__ __launch_bounds__(1024) void damp_stats_kernel(float* __restrict__ H, int64_t n,
                                                          uint8_t* __restrict__ dead, float damp,
                                                          double* __restrict__ lam_out) {
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    float d = H[i * n + i];
    const bool z = d == 0.0f;
    dead[i] = z ? 1 : 0;
    if (z) {
      d = 1.0f;
      H[i * n + i] = 1.0f;
    }
    s += (double)d;
  }
  __shared__ double red[1024];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) lam_out[0] = (double)damp * (red[0] / (double)n);
}

__global__ void add_diag_kernel(float* __restrict__ H, int64_t n, const double* __restrict__ lam) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) H[i * n + i] = (float)((double)H[i * n + i] + lam[0]);
}

// Diagonal block at rows/cols [s0, s0 + NB): factor A22 = R22 R22^T (R22 upper) and
// store U22 = R22^-1 in its place (zeros below the diagonal).  One wave of 64 lanes,
// so a barrier costs almost nothing:
//   factor: lane i holds row i; column j of the elimination goes through LDS and is
//           read back by every lane (broadcast), A[i][k] -= a_ij a_kj / p (i <= k < j);
//   inverse: R is staged in LDS; lane c back-substitutes column c of U = R^-1,
//           U[i][c] = -(sum_{k > i} R[i][k] U[k][c]) / R[i][i], U[c][c] = 1 / R[c][c].
__global__ __launch_bounds__(NB) void diag_factor_inverse_kernel(float* __restrict__ H, int64_t n,
                                                                 int64_t s0, int* __restrict__ flag) {
  __shared__ float col[NB];
  __shared__ float R[NB * LD];
  const int l = threadIdx.x;
  // coalesced load of the block's upper triangle into LDS, then row l into registers
  for (int i = 0; i < NB; ++i) R[i * LD + l] = l >= i ? H[(s0 + i) * n + s0 + l] : 0.0f;
  __syncthreads();
  float a[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) a[k] = R[l * LD + k];
  bool bad = false;
#pragma unroll
  for (int j = NB - 1; j >= 0; --j) {
    col[l] = a[j];
    __syncthreads();
    const float p = col[j];
    const float rs = rsqrtf(p);
    const float f = a[j] * (1.0f / p);
#pragma unroll
    for (int k = 0; k < j; ++k) {
      const float upd = fmaf(-f, col[k], a[k]);
      a[k] = k >= l ? upd : a[k];
    }
    a[j] = l < j ? a[j] * rs : (l == j ? p * rs : a[j]);
    bad |= (l == j) && !(p > 0.0f);
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) R[l * LD + k] = a[k];
  __syncthreads();
  float x[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) x[i] = 0.0f;
#pragma unroll
  for (int i = NB - 1; i >= 0; --i) {
    float acc = 0.0f;
#pragma unroll
    for (int k = i + 1; k < NB; ++k) acc = fmaf(R[i * LD + k], x[k], acc);
    const float rinv = 1.0f / R[i * LD + i];
    x[i] = i == l ? rinv : (i < l ? -acc * rinv : 0.0f);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) H[(s0 + i) * n + s0 + l] = x[i];
  if (bad) atomicOr(flag, 1);
}

// Clears the strictly lower triangle (row k, columns j < k).
__global__ void zero_lower_kernel(float* __restrict__ H, int64_t n) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t k = blockIdx.y;
  if (j < k) H[k * n + j] = 0.0f;
}

}  // namespace

// Copies HX into the workspace matrix F, damps it, factors it (H_d = R R^T) and
// replaces R by U = R^-1 (upper triangle; the strictly lower triangle is zeroed).
// T is scratch of n * n / 4 floats.
kq_status damp_and_factor(const float* HX, float* F, float* T, uint8_t* dead, double* lam,
                          int* flag, int64_t n, float damp, hipStream_t s) {
  if (n % NB != 0) return fail(KQ_ESHAPE, "factorization needs n %% %d == 0", NB);
  KQ_HIP(hipMemcpyAsync(F, HX, n * n * sizeof(float), hipMemcpyDeviceToDevice, s));
  damp_stats_kernel<<<1, 1024, 0, s>>>(F, n, dead, damp, lam);
  KQ_LAUNCHED("damp_stats_kernel");
  add_diag_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s>>>(F, n, lam);
  KQ_LAUNCHED("add_diag_kernel");
  // reverse Cholesky; diagonal blocks are left holding U_JJ = R_JJ^-1
  for (int64_t s0 = n - NB; s0 >= 0; s0 -= NB) {
    diag_factor_inverse_kernel<<<1, NB, 0, s>>>(F, n, s0, flag);
    KQ_LAUNCHED("diag_factor_inverse_kernel");
    if (s0 == 0) break;
    // R12 = A12 R22^-T = A12 U22^T  (in place; each row tile reads its 64 columns first)
    GemmArgs p{};
    p.M = s0; p.N = NB; p.K = NB;
    p.A = F + s0; p.lda = n; p.B = F + s0 * n + s0; p.ldb = n; p.transB = true;
    p.C = F + s0; p.ldc = n; p.alpha = 1.0f; p.split_k = 1;
    KQ_TRY(gemm_f32(p, s));
    // A11 -= R12 R12^T (upper tiles)
    GemmArgs g{};
    g.M = s0; g.N = s0; g.K = NB;
    g.A = F + s0; g.lda = n; g.B = F + s0; g.ldb = n; g.transB = true;
    g.C = F; g.ldc = n;
    g.alpha = -1.0f; g.accumulate = true; g.upper_only = true; g.split_k = 1;
    KQ_TRY(gemm_f32(g, s));
  }
  dim3 zgrid((unsigned)ceil_div(n, 256), (unsigned)n);
  zero_lower_kernel<<<zgrid, dim3(256), 0, s>>>(F, n);
  KQ_LAUNCHED("zero_lower_kernel");
  // U = R^-1 by recursive doubling over the diagonal blocks:
  //   inv([[A, B], [0, D]]) = [[A^-1, -A^-1 B D^-1], [0, D^-1]]
  // Neighbouring blocks are paired level by level; the pairs of one level with equal
  // sizes form one batched product.
  struct Blk { int64_t o, sz; };
  int64_t nblk = n / NB;
  Blk* blocks = new Blk[nblk];
  Blk* next = new Blk[nblk];
  for (int64_t b = 0; b < nblk; ++b) blocks[b] = Blk{b * NB, NB};
  kq_status st = KQ_OK;
  while (nblk > 1 && st == KQ_OK) {
    int64_t nn = 0;
    int64_t p = 0;
    while (p + 1 < nblk && st == KQ_OK) {
      // maximal run of consecutive pairs with the same sizes
      const int64_t sa = blocks[p].sz, sd = blocks[p + 1].sz;
      int64_t run = 1;
      while (p + 2 * run + 1 < nblk && blocks[p + 2 * run].sz == sa && blocks[p + 2 * run + 1].sz == sd)
        ++run;
      const int64_t oa = blocks[p].o, od = blocks[p + 1].o;
      const int64_t diag_stride = (sa + sd) * (n + 1);
      GemmArgs t{};
      t.M = sa; t.N = sd; t.K = sa;
      t.A = F + oa * n + oa; t.lda = n; t.a_upper = true;
      t.B = F + oa * n + od; t.ldb = n;
      t.C = T; t.ldc = sd; t.alpha = 1.0f; t.split_k = 1;
      t.batch = (int)run; t.strideA = diag_stride; t.strideB = diag_stride; t.strideC = sa * sd;
      st = gemm_f32(t, s);
      if (st != KQ_OK) break;
      GemmArgs x{};
      x.M = sa; x.N = sd; x.K = sd;
      x.A = T; x.lda = sd;
      x.B = F + od * n + od; x.ldb = n; x.b_upper = true;
      x.C = F + oa * n + od; x.ldc = n; x.alpha = -1.0f; x.split_k = 1;
      x.batch = (int)run; x.strideA = sa * sd; x.strideB = diag_stride; x.strideC = diag_stride;
      st = gemm_f32(x, s);
      for (int64_t r = 0; r < run; ++r) next[nn++] = Blk{blocks[p + 2 * r].o, sa + sd};
      p += 2 * run;
    }
    if (p < nblk) next[nn++] = blocks[p];
    Blk* tmp = blocks; blocks = next; next = tmp;
    nblk = nn;
  }
  delete[] blocks;
  delete[] next;
  return st;
}

}  // namespace kq
