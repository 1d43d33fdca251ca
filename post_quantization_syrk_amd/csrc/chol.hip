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

// Factor the diagonal block at rows/cols [s0, s0 + nb) in place: A22 = R22 R22^T.
__global__ __launch_bounds__(256) void diag_factor_kernel(float* __restrict__ H, int64_t n,
                                                          int64_t s0, int nb,
                                                          int* __restrict__ flag) {
  __shared__ float A[NB * LD];
  __shared__ int bad;
  const int t = threadIdx.x;
  if (t == 0) bad = 0;
  for (int e = t; e < nb * nb; e += 256) {
    const int i = e / nb, k = e % nb;
    A[i * LD + k] = i <= k ? H[(s0 + i) * n + s0 + k] : 0.0f;
  }
  __syncthreads();
  for (int j = nb - 1; j >= 0; --j) {
    const float p = A[j * LD + j];
    const float d = sqrtf(p);
    if (t == 0 && !(p > 0.0f)) bad = 1;
    if (t < j) A[t * LD + j] /= d;
    __syncthreads();
    if (t == 0) A[j * LD + j] = d;
    // A[i][k] -= R[i][j] R[k][j] for i <= k < j
    for (int e = t; e < j * j; e += 256) {
      const int i = e / j, k = e % j;
      if (i <= k) A[i * LD + k] -= A[i * LD + j] * A[k * LD + j];
    }
    __syncthreads();
  }
  for (int e = t; e < nb * nb; e += 256) {
    const int i = e / nb, k = e % nb;
    if (i <= k) H[(s0 + i) * n + s0 + k] = A[i * LD + k];
  }
  if (t == 0 && bad) atomicOr(flag, 1);
}

// Rows r < s0: solve x R22^T = h (h = H[r, s0:s0+nb]) and store x over h.
__global__ __launch_bounds__(256) void panel_solve_kernel(float* __restrict__ H, int64_t n,
                                                          int64_t s0) {
  __shared__ float R[NB * LD];
  const int t = threadIdx.x;
  for (int e = t; e < NB * NB; e += 256) {
    const int i = e / NB, k = e % NB;
    R[i * LD + k] = i <= k ? H[(s0 + i) * n + s0 + k] : 0.0f;
  }
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * 256 + t;
  if (r >= s0) return;
  float* row = H + r * n + s0;
  float x[NB];
#pragma unroll
  for (int k = 0; k < NB; k += 4) {
    float4 v = *(const float4*)(row + k);
    x[k] = v.x; x[k + 1] = v.y; x[k + 2] = v.z; x[k + 3] = v.w;
  }
  // h_j = sum_{k >= j} x_k R[j][k]  ->  x_j = (h_j - sum_{k > j} x_k R[j][k]) / R[j][j]
#pragma unroll
  for (int j = NB - 1; j >= 0; --j) {
    float acc = x[j];
#pragma unroll
    for (int k = j + 1; k < NB; ++k) acc -= x[k] * R[j * LD + k];
    x[j] = acc / R[j * LD + j];
  }
#pragma unroll
  for (int k = 0; k < NB; k += 4) *(float4*)(row + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
}

// Clears the strictly lower triangle (row k, columns j < k).
__global__ void zero_lower_kernel(float* __restrict__ H, int64_t n) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t k = blockIdx.y;
  if (j < k) H[k * n + j] = 0.0f;
}

// In-place inverse of every 64 x 64 upper-triangular diagonal block (one block per
// workgroup): column c of X = R^-1 by back substitution, X[c][c] = 1 / R[c][c],
// X[i][c] = -(sum_{k=i+1..c} R[i][k] X[k][c]) / R[i][i] for i < c.
__global__ __launch_bounds__(NB) void diag_inverse_kernel(float* __restrict__ H, int64_t n) {
  __shared__ float R[NB * LD];
  __shared__ float X[NB * LD];
  const int64_t s0 = (int64_t)blockIdx.x * NB;
  const int c = threadIdx.x;
  for (int i = 0; i < NB; ++i) {
    R[i * LD + c] = i <= c ? H[(s0 + i) * n + s0 + c] : 0.0f;
    X[i * LD + c] = 0.0f;
  }
  __syncthreads();
  X[c * LD + c] = 1.0f / R[c * LD + c];
  for (int i = c - 1; i >= 0; --i) {
    float acc = 0.0f;
    for (int k = i + 1; k <= c; ++k) acc += R[i * LD + k] * X[k * LD + c];
    X[i * LD + c] = -acc / R[i * LD + i];
  }
  for (int i = 0; i <= c; ++i) H[(s0 + i) * n + s0 + c] = X[i * LD + c];
}

}  // namespace

// Copies HX into the workspace matrix F, damps it, factors it (H_d = R R^T) and
// replaces R by U = R^-1 (upper triangle; the strictly lower triangle is zeroed).
// T is scratch of n * NB floats.
kq_status damp_and_factor(const float* HX, float* F, float* T, uint8_t* dead, double* lam,
                          int* flag, int64_t n, float damp, hipStream_t s) {
  if (n % NB != 0) return fail(KQ_ESHAPE, "factorization needs n %% %d == 0", NB);
  KQ_HIP(hipMemcpyAsync(F, HX, n * n * sizeof(float), hipMemcpyDeviceToDevice, s));
  damp_stats_kernel<<<1, 1024, 0, s>>>(F, n, dead, damp, lam);
  KQ_LAUNCHED("damp_stats_kernel");
  add_diag_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s>>>(F, n, lam);
  KQ_LAUNCHED("add_diag_kernel");
  for (int64_t s0 = n - NB; s0 >= 0; s0 -= NB) {
    diag_factor_kernel<<<1, 256, 0, s>>>(F, n, s0, NB, flag);
    KQ_LAUNCHED("diag_factor_kernel");
    if (s0 == 0) break;
    panel_solve_kernel<<<dim3((unsigned)ceil_div(s0, 256)), dim3(256), 0, s>>>(F, n, s0);
    KQ_LAUNCHED("panel_solve_kernel");
    GemmArgs g{};
    g.M = s0; g.N = s0; g.K = NB;
    g.A = F + s0; g.lda = n; g.transA = false;
    g.B = F + s0; g.ldb = n; g.transB = true;
    g.C = F; g.ldc = n;
    g.alpha = -1.0f; g.accumulate = true; g.upper_only = true; g.split_k = 1;
    KQ_TRY(gemm_f32(g, s));
  }
  dim3 zgrid((unsigned)ceil_div(n, 256), (unsigned)n);
  zero_lower_kernel<<<zgrid, dim3(256), 0, s>>>(F, n);
  KQ_LAUNCHED("zero_lower_kernel");
  // U = R^-1
  diag_inverse_kernel<<<dim3((unsigned)(n / NB)), dim3(NB), 0, s>>>(F, n);
  KQ_LAUNCHED("diag_inverse_kernel");
  for (int64_t j0 = NB; j0 < n; j0 += NB) {
    // T = U[<j0, <j0] R[<j0, J]   (U upper: row tile i only needs k >= its first row)
    GemmArgs g{};
    g.M = j0; g.N = NB; g.K = j0;
    g.A = F; g.lda = n; g.B = F + j0; g.ldb = n;
    g.C = T; g.ldc = NB; g.alpha = 1.0f; g.split_k = 1; g.a_upper = true;
    KQ_TRY(gemm_f32(g, s));
    // U[<j0, J] = -T U_JJ
    GemmArgs h{};
    h.M = j0; h.N = NB; h.K = NB;
    h.A = T; h.lda = NB; h.B = F + j0 * n + j0; h.ldb = n;
    h.C = F + j0; h.ldc = n; h.alpha = -1.0f; h.split_k = 1;
    KQ_TRY(gemm_f32(h, s));
  }
  return KQ_OK;
}

}  // namespace kq
