// Damping, the reverse-order Cholesky factor of the processed H_X, and the factors GPTQ's
// blocked error feedback uses.
//
// GPTQ, which KronQ runs as its base quantizer (KronQ README, "Mapping paper
// results to flags": GPTQ is the baseline with no extra flags; the opening
// section: KronQ extends GPTQ/GPTAQ), rounds column by column through
// U = chol_upper(H_d^-1), H_d = H_X + lambda I, lambda = damp * mean(diag H_X).
// Here H_d = R R^T with R upper triangular is factored from the bottom-right
// corner up; then U = R^-1, since U^T U = R^-T R^-1 = H_d^-1 and U is upper
// with a positive diagonal.
//
// Reverse Cholesky, 64-column blocks from the last one up, two launches per block:
//   panel:   R12 = A12 U22^T            (U22 = R22^-1 from the previous launch; fp32 MFMA)
//   update:  A11 -= R12 R12^T           (fp32 MFMA, upper 128 x 128 tiles), while one extra
//            workgroup updates the next diagonal block privately and factors it (one wave:
//            R22 R22^T = A22; then U22 = R22^-1 by recursive doubling on all four waves),
//            so the serial chain of small factorizations overlaps the bulk updates.
// Only the diagonal blocks of U are formed.  GPTQ's feedback into block J needs
// U[<J, J] = -U[<J,<J] R[<J, J] U_JJ only through E[:, <J] U[<J, J], and
// E[:, <J] U[<J,<J] = (W - Qhat)[:, <J] (the rounding error so far, in the layer's own
// basis), so the factor kept for block J is P[<J, J] = R[<J, J] U_JJ.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int NB = 64;

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

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int LB = 68;    // row stride of the 64 x 64 blocks the leaf works on (LDS)
constexpr int LP = 65;    // row stride of the MFMA operand slabs in LDS

// Orders one wave's LDS accesses between lanes (a wave's LDS operations run in order; this
// only keeps the compiler from moving them across).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Leaf factorization, run by one wave: Ab (LDS, 64 x 64, row stride LB) holds the upper
// triangle of a diagonal block A' (entries below the diagonal are ignored).  Factors
// A' = R R^T from the last column up (R upper): lane l holds row l of A' (becoming row l of
// R).  Step j: the lanes publish column j (col[]), p = A'_jj, R_jj = sqrt(p);
// A'_lk -= A'_lj A'_kj / p for k < j (every lane updates its whole row; the lower part it
// also touches is never read); R_lj = A'_lj / R_jj goes to Rl and 1 / R_jj to rsq.  Rl's
// entries below the diagonal are left undefined.  Sets *flag on a non-positive pivot.
__device__ __forceinline__ void leaf_factor(const float* Ab, float* Rl, float* col, float* rsq,
                                            int* flag) {
  const int l = threadIdx.x & 63;
  float a[64];
#pragma unroll
  for (int k = 0; k < 64; k += 4) {
    const float4 v = *(const float4*)(Ab + l * LB + k);
    a[k] = v.x; a[k + 1] = v.y; a[k + 2] = v.z; a[k + 3] = v.w;
  }
  bool bad = false;
#pragma unroll
  for (int j = 63; j >= 0; --j) {
    col[l] = a[j];
    wave_sync();
    const float p = col[j];
    const float rs = rsqrtf(p);
    const float f = a[j] * (rs * rs);
#pragma unroll
    for (int k = 0; k < j; ++k) a[k] = fmaf(-f, col[k], a[k]);
    a[j] *= rs;
    Rl[l * LB + j] = a[j];
    rsq[j] = rs;
    bad |= (l == j) & !(p > 0.0f);
    wave_sync();
  }
  if (bad) atomicOr(flag, 1);
}

// U = R^-1 for the 64 x 64 upper R in Rl (only entries on or above the diagonal are read;
// rsq[j] = 1 / R_jj), by recursive doubling, with all 4 waves of the workgroup:
//   16 x 16 diagonal blocks by back substitution (one wave each, lane = column),
//   then inv([[A, B], [0, D]]) = [[A^-1, -A^-1 B D^-1], [0, D^-1]] at 32 and 64
//   (v_mfma_f32_16x16x4f32).  Ul (64 x LB) receives U with zeros below the diagonal;
//   Ts is scratch of 32 x LB floats.  Contains workgroup barriers: every thread calls it.
__device__ __forceinline__ void leaf_inverse(const float* Rl, const float* rsq, float* Ul,
                                             float* Ts) {
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int r16 = lane & 15, k4 = lane >> 4;
  for (int q = t; q < 64 * LB; q += 256) Ul[q] = 0.0f;
  __syncthreads();
  {
    // diagonal block w: x = column c of its inverse
    const int b = 16 * w, c = r16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.0f;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      float sum = 0.0f;
#pragma unroll
      for (int k = i + 1; k < 16; ++k) sum = fmaf(Rl[(b + i) * LB + b + k], x[k], sum);
      const float r = rsq[b + i];
      const float v = -r * sum;
      x[i] = i == c ? r : (i < c ? v : 0.0f);
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Ul[(b + i) * LB + b + c] = x[i];
    }
  }
  __syncthreads();
  if (w == 0 || w == 2) {
    // pair (b, b+16): U[b.., b+16..] = -(U[b.., b..] R[b.., b+16..]) U[b+16.., b+16..]
    const int b = 16 * w;
    float* T = Ts + (w >> 1) * 16 * LB;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < 16; kk += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ul[(b + r16) * LB + b + kk + k4],
                                                 Rl[(b + kk + k4) * LB + b + 16 + r16], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) T[(4 * k4 + r) * LB + r16] = acc[r];
    wave_sync();
    f32x4 acc2 = f32x4{};
#pragma unroll
    for (int kk = 0; kk < 16; kk += 4)
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(T[r16 * LB + kk + k4],
                                                  Ul[(b + 16 + kk + k4) * LB + b + 16 + r16], acc2,
                                                  0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) Ul[(b + 4 * k4 + r) * LB + b + 16 + r16] = -acc2[r];
  }
  __syncthreads();
  // halves (0, 32): U[0..32, 32..64] = -(U[0..32, 0..32] R[0..32, 32..64]) U[32.., 32..];
  // wave w forms the 16 x 16 quadrant (qi, qj)
  const int qi = w >> 1, qj = w & 1;
  f32x4 acc = f32x4{};
#pragma unroll
  for (int kk = 0; kk < 32; kk += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ul[(16 * qi + r16) * LB + kk + k4],
                                               Rl[(kk + k4) * LB + 32 + 16 * qj + r16], acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) Ts[(16 * qi + 4 * k4 + r) * LB + 16 * qj + r16] = acc[r];
  __syncthreads();
  f32x4 acc2 = f32x4{};
#pragma unroll
  for (int kk = 0; kk < 32; kk += 4)
    acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ts[(16 * qi + r16) * LB + kk + k4],
                                                Ul[(32 + kk + k4) * LB + 32 + 16 * qj + r16], acc2,
                                                0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) Ul[(16 * qi + 4 * k4 + r) * LB + 32 + 16 * qj + r16] = -acc2[r];
  __syncthreads();
}

// LDS for a leaf: X (64 x LB: A', then U) and Y (64 x LB for R, 64 + 64 for the column and
// 1 / R_jj, 32 x LB scratch).
constexpr int LEAF_Y = 64 * LB + 128 + 32 * LB;

// Factor + invert the diagonal block held in X; U goes to out (64 x 64 row-major).
// Every thread of the 256-thread workgroup calls it.
__device__ __forceinline__ void leaf(float* X, float* Y, float* __restrict__ out, int* flag) {
  float* Rl = Y;
  float* col = Y + 64 * LB;
  float* rsq = col + 64;
  float* Ts = rsq + 64;
  if (threadIdx.x < 64) leaf_factor(X, Rl, col, rsq, flag);
  __syncthreads();
  leaf_inverse(Rl, rsq, X, Ts);
  for (int q = threadIdx.x; q < 64 * 64; q += 256) out[q] = X[(q >> 6) * LB + (q & 63)];
}

// The last diagonal block [s0, s0 + 64), factored on its own.
__global__ __launch_bounds__(256) void leaf_kernel(const float* __restrict__ F, int64_t n,
                                                   int64_t s0, float* __restrict__ Uout,
                                                   int* __restrict__ flag) {
  __shared__ __attribute__((aligned(16))) float X[64 * LB];
  __shared__ __attribute__((aligned(16))) float Y[LEAF_Y];
  for (int q = threadIdx.x; q < 64 * 64; q += 256)
    X[(q >> 6) * LB + (q & 63)] = F[(s0 + (q >> 6)) * n + s0 + (q & 63)];
  __syncthreads();
  leaf(X, Y, Uout, flag);
}

// Panel R12 = A12 U22^T for rows [128 b, 128 b + 128) of [0, s0) and columns [s0, s0 + 64),
// in place (each workgroup reads and writes its own rows).  U22 = R22^-1 comes from the
// block buffer.  4 waves, each 32 rows x 64 columns of v_mfma_f32_32x32x2f32.
__global__ __launch_bounds__(256) void panel_kernel(float* __restrict__ F, int64_t n, int64_t s0,
                                                    const float* __restrict__ U22) {
  __shared__ float As[128 * LP];
  __shared__ float Us[64 * LP];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 128;
  for (int q = t; q < 128 * 16; q += 256) {
    const int r = q >> 4, c4 = (q & 15) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + r < s0) v = *(const float4*)(F + (r0 + r) * n + s0 + c4);
    float* d = As + r * LP + c4;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  for (int q = t; q < 64 * 16; q += 256) {
    const int r = q >> 4, c4 = (q & 15) * 4;
    const float4 v = *(const float4*)(U22 + r * 64 + c4);
    float* d = Us + r * LP + c4;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();
  const int lane = t & 63, w = t >> 6, l32 = lane & 31, kh = lane >> 5;
  f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float av[16], bv[16][2];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 32 * h + 2 * kk + kh;
      av[kk] = As[(32 * w + l32) * LP + k];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) bv[kk][jb] = Us[(32 * jb + l32) * LP + k];   // U22[c][k]
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk], bv[kk][jb], acc[jb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = r0 + 32 * w + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (row < s0) F[row * n + s0 + 32 * jb + l32] = acc[jb][r];
    }
}

// Trailing update A11 -= R12 R12^T, R12 = F[0:s0, s0:s0+64], over the upper 128 x 128 tiles
// of [0, s0)^2.  The next diagonal block D = [s0-64, s0)^2 is left alone by these tiles:
// workgroup 0 instead forms D - R_D R_D^T (R_D = rows s0-64.. of R12) privately and factors
// it (leaf), so the next block's factorization overlaps the bulk update.  Its U goes to Unext.
// Tiles: 4 waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x2f32 blocks), K = 64 in one LDS stage;
// the tile's old values are loaded first so their latency overlaps the operand loads.
__global__ __launch_bounds__(256) void update_kernel(float* __restrict__ F, int64_t n, int64_t s0,
                                                     float* __restrict__ Unext,
                                                     int* __restrict__ flag) {
  __shared__ __attribute__((aligned(16))) float As[128 * LP];
  __shared__ __attribute__((aligned(16))) float Bs[128 * LP];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, l32 = lane & 31, kh = lane >> 5;
  const int64_t d0 = s0 - 64;
  if (blockIdx.x == 0) {
    // R_D (64 x 64) into As (stride LP); D into Bs (stride LB, the leaf's layout)
    for (int q = t; q < 64 * 16; q += 256) {
      const int r = q >> 4, c4 = (q & 15) * 4;
      const float4 v = *(const float4*)(F + (d0 + r) * n + s0 + c4);
      float* d = As + r * LP + c4;
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      *(float4*)(Bs + r * LB + c4) = *(const float4*)(F + (d0 + r) * n + d0 + c4);
    }
    __syncthreads();
    // wave (wi, wj) forms the 32 x 32 block (wi, wj) of D - R_D R_D^T
    const int wi = w >> 1, wj = w & 1;
    f32x16 acc = f32x16{};
#pragma unroll 8
    for (int k = 0; k < 64; k += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[(32 * wi + l32) * LP + k + kh],
                                                 As[(32 * wj + l32) * LP + k + kh], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * wi + 8 * (r >> 2) + 4 * kh + (r & 3);
      float* d = Bs + row * LB + 32 * wj + l32;
      *d = *d - acc[r];
    }
    __syncthreads();
    leaf(Bs, As, Unext, flag);
    return;
  }
  // upper tile (tm, tn), tm <= tn, enumerated row by row
  const int m = (int)((s0 + 127) / 128);
  int idx = blockIdx.x - 1, tm = 0;
  while (idx >= m - tm) { idx -= m - tm; ++tm; }
  const int tn = tm + idx;
  const int64_t i0 = (int64_t)tm * 128, j0 = (int64_t)tn * 128;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  // this lane's tile entries: rows rbase + 32 i + 8 (r / 4) + r % 4, columns cbase + 32 j
  const int64_t rbase = i0 + wm + 4 * kh, cbase = j0 + wn + l32;
  const float* cptr = F + rbase * n + cbase;
  const int rlim = (int)min((int64_t)128, s0 - rbase), clim = (int)min((int64_t)128, s0 - cbase);
  float cv[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ro = 32 * i + 8 * (r >> 2) + (r & 3);
        cv[i][j][r] = (ro < rlim && 32 * j < clim) ? cptr[(int64_t)ro * n + 32 * j] : 0.0f;
      }
  const bool same = tm == tn;
  for (int q = t; q < 128 * 16; q += 256) {
    const int r = q >> 4, c4 = (q & 15) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 + r < s0) v = *(const float4*)(F + (i0 + r) * n + s0 + c4);
    float* d = As + r * LP + c4;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    if (!same) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + r < s0) u = *(const float4*)(F + (j0 + r) * n + s0 + c4);
      float* e = Bs + r * LP + c4;
      e[0] = u.x; e[1] = u.y; e[2] = u.z; e[3] = u.w;
    }
  }
  __syncthreads();
  const float* Bp = same ? As : Bs;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  // two halves of 32 k; each half's operands are read before its multiplies
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float av[16][2], bv[16][2];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 32 * h + 2 * kk + kh;
#pragma unroll
      for (int i = 0; i < 2; ++i) av[kk][i] = As[(wm + 32 * i + l32) * LP + k];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[kk][j] = Bp[(wn + 32 * j + l32) * LP + k];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  float* optr = F + rbase * n + cbase;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ro = 32 * i + 8 * (r >> 2) + (r & 3);
        const bool in_d = rbase + ro >= d0 && cbase + 32 * j >= d0;
        if (ro < rlim && 32 * j < clim && !in_d)
          optr[(int64_t)ro * n + 32 * j] = cv[i][j][r] - acc[i][j][r];
      }
}

// Clears the strictly lower triangle and moves each diagonal block's U_JJ from the block
// buffer into place.
__global__ void finalize_kernel(float* __restrict__ F, int64_t n, const float* __restrict__ Ubuf) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t k = blockIdx.y;
  if (j >= n) return;
  const int64_t bk = k >> 6, bj = j >> 6;
  if (bj == bk) F[k * n + j] = Ubuf[bk * 4096 + (k & 63) * 64 + (j & 63)];
  else if (j < k) F[k * n + j] = 0.0f;
}

// For GPTQ blocks of 128 columns, the 128 x 128 diagonal block of U = R^-1 from its two
// 64-blocks: U_ab = -U_a R_ab U_b (written over R_ab).  One workgroup per 128-block; each wave
// forms a 32 x 32 quadrant of each product (v_mfma_f32_32x32x2f32).
__global__ __launch_bounds__(256) void ujj128_kernel(float* __restrict__ F, int64_t n) {
  __shared__ float Ua[64 * LP];
  __shared__ float Rab[64 * LP];
  __shared__ float Ub[64 * LP];
  __shared__ float Ts[64 * LP];
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  const int64_t a0 = (int64_t)blockIdx.x * 128, b0 = a0 + 64;
  for (int q = t; q < 64 * 64; q += 256) {
    const int r = q >> 6, c = q & 63;
    Ua[r * LP + c] = F[(a0 + r) * n + a0 + c];
    Rab[r * LP + c] = F[(a0 + r) * n + b0 + c];
    Ub[r * LP + c] = F[(b0 + r) * n + b0 + c];
  }
  __syncthreads();
  const int wi = w >> 1, wj = w & 1;
  f32x16 acc = f32x16{};
#pragma unroll 8
  for (int k = 0; k < 64; k += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ua[(32 * wi + l32) * LP + k + kh],
                                               Rab[(k + kh) * LP + 32 * wj + l32], acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) Ts[(32 * wi + 8 * (r >> 2) + 4 * kh + (r & 3)) * LP + 32 * wj + l32] = acc[r];
  __syncthreads();
  f32x16 acc2 = f32x16{};
#pragma unroll 8
  for (int k = 0; k < 64; k += 2)
    acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(Ts[(32 * wi + l32) * LP + k + kh],
                                                Ub[(k + kh) * LP + 32 * wj + l32], acc2, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    F[(a0 + 32 * wi + 8 * (r >> 2) + 4 * kh + (r & 3)) * n + b0 + 32 * wj + l32] = -acc2[r];
}

// GPTQ feedback factors P[<J, J] = R[<J, J] U_JJ for every column block J of width B, in place
// over R (one workgroup per (row tile i, block J) with i < J; tiles of B x B, K = B).
// Waves: B = 128, 64 x 64 each (2 x 2 MFMA blocks); B = 64, 32 x 32 each.
template <int B>
__global__ __launch_bounds__(256) void pmat_kernel(float* __restrict__ F, int64_t n) {
  constexpr int LDQ = B + 1;
  constexpr int WT = B / 2;           // wave tile edge
  constexpr int NBK = WT / 32;        // 32 x 32 blocks per wave edge
  __shared__ float Rs[B * LDQ];
  __shared__ float Us[B * LDQ];
  int idx = blockIdx.x, J = 1;
  while (idx >= J) { idx -= J; ++J; }
  const int64_t r0 = (int64_t)idx * B, c0 = (int64_t)J * B;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  for (int q = t; q < B * B / 4; q += 256) {
    const int r = q / (B / 4), c4 = 4 * (q % (B / 4));
    const float4 v = *(const float4*)(F + (r0 + r) * n + c0 + c4);
    const float4 u = *(const float4*)(F + (c0 + r) * n + c0 + c4);
    float* d = Rs + r * LDQ + c4;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    float* e = Us + r * LDQ + c4;
    // U_JJ is upper triangular; entries below its diagonal are not U's
    e[0] = c4 + 0 >= r ? u.x : 0.0f;
    e[1] = c4 + 1 >= r ? u.y : 0.0f;
    e[2] = c4 + 2 >= r ? u.z : 0.0f;
    e[3] = c4 + 3 >= r ? u.w : 0.0f;
  }
  __syncthreads();
  const int wm = (w >> 1) * WT, wn = (w & 1) * WT;
  f32x16 acc[NBK][NBK];
#pragma unroll
  for (int i = 0; i < NBK; ++i)
#pragma unroll
    for (int j = 0; j < NBK; ++j) acc[i][j] = f32x16{};
#pragma unroll
  for (int h = 0; h < B / 32; ++h) {
    float av[16][NBK], bv[16][NBK];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 32 * h + 2 * kk + kh;
#pragma unroll
      for (int i = 0; i < NBK; ++i) av[kk][i] = Rs[(wm + 32 * i + l32) * LDQ + k];
#pragma unroll
      for (int j = 0; j < NBK; ++j) bv[kk][j] = Us[k * LDQ + wn + 32 * j + l32];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int j = 0; j < NBK; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NBK; ++i)
#pragma unroll
    for (int j = 0; j < NBK; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        F[(r0 + wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3)) * n + c0 + wn + 32 * j + l32] =
            acc[i][j][r];
}

}  // namespace

// Copies HX into the workspace matrix F, damps it and factors it (H_d = R R^T).  On return F
// holds, above its B x B diagonal blocks, GPTQ's feedback factors P = R[<J, J] U_JJ, and in
// those blocks U_JJ (U = R^-1 = chol_upper(H_d^-1)); the strictly lower triangle is zero.
// T is scratch of 64 n floats.
kq_status damp_and_factor(const float* HX, float* F, float* T, uint8_t* dead, double* lam,
                          int* flag, int64_t n, float damp, int B, hipStream_t s) {
  if (n % NB != 0) return fail(KQ_ESHAPE, "factorization needs n %% %d == 0", NB);
  if ((B != 64 && B != 128) || n % B != 0) return fail(KQ_ESHAPE, "bad GPTQ block %d", B);
  KQ_HIP(hipMemcpyAsync(F, HX, n * n * sizeof(float), hipMemcpyDeviceToDevice, s));
  damp_stats_kernel<<<1, 1024, 0, s>>>(F, n, dead, damp, lam);
  KQ_LAUNCHED("damp_stats_kernel");
  add_diag_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s>>>(F, n, lam);
  KQ_LAUNCHED("add_diag_kernel");
  // reverse Cholesky.  The diagonal blocks' U_JJ = R_JJ^-1 are kept in the block buffer T
  // (64 n floats); F holds A, then R above the diagonal blocks.
  float* Ubuf = T;
  const int64_t nb = n / NB;
  leaf_kernel<<<1, 256, 0, s>>>(F, n, n - NB, Ubuf + (nb - 1) * 4096, flag);
  KQ_LAUNCHED("leaf_kernel");
  for (int64_t s0 = n - NB; s0 >= NB; s0 -= NB) {
    panel_kernel<<<dim3((unsigned)ceil_div(s0, 128)), dim3(256), 0, s>>>(F, n, s0,
                                                                        Ubuf + (s0 / NB) * 4096);
    KQ_LAUNCHED("panel_kernel");
    const int64_t m = ceil_div(s0, 128);
    const int64_t tiles = s0 > NB ? m * (m + 1) / 2 : 0;
    update_kernel<<<dim3((unsigned)(1 + tiles)), dim3(256), 0, s>>>(
        F, n, s0, Ubuf + (s0 / NB - 1) * 4096, flag);
    KQ_LAUNCHED("update_kernel");
  }
  dim3 zgrid((unsigned)ceil_div(n, 256), (unsigned)n);
  finalize_kernel<<<zgrid, dim3(256), 0, s>>>(F, n, Ubuf);
  KQ_LAUNCHED("finalize_kernel");
  // GPTQ's feedback factors: the B x B diagonal blocks of U and P[<J, J] = R[<J, J] U_JJ
  if (B == 128) {
    ujj128_kernel<<<dim3((unsigned)(n / 128)), dim3(256), 0, s>>>(F, n);
    KQ_LAUNCHED("ujj128_kernel");
  }
  const int64_t nbl = n / B;
  const int64_t pairs = nbl * (nbl - 1) / 2;
  if (pairs > 0) {
    if (B == 128) pmat_kernel<128><<<dim3((unsigned)pairs), dim3(256), 0, s>>>(F, n);
    else pmat_kernel<64><<<dim3((unsigned)pairs), dim3(256), 0, s>>>(F, n);
    KQ_LAUNCHED("pmat_kernel");
  }
  return KQ_OK;
}

}  // namespace kq
