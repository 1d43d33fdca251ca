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
// Reverse Cholesky, 64-column blocks from the last one up, one launch per block.  With A12
// the current column block above the diagonal and M = A22^-1 = U22^T U22 (from the previous
// block's leaf), the block's panel factor is Z = A12 M (= R12 U22), kept transposed in the
// free lower triangle, and the trailing update is A11 -= Z A12^T.  That update is split in
// two: the columns are grouped in super-blocks of 1024 (aligned to 0), and a step updates
// only the columns of its own super-block that are still to come (every row above them:
// 128 x 128 fp32 MFMA tiles, each forming Z for its rows); the rest of A11, left of the
// super-block, takes the super-block's whole rank-1024 update at once when the super-block
// is done, as one plain product A12 Z^T of the super-block's columns with the Z^T rows of the
// lower triangle (equal to Z A12^T, the update being symmetric).  So the leading matrix is
// read and written once per super-block rather than once per block (matrices that fit the
// last-level cache, 64 MB at 4096 wide, are one super-block: there the split only adds to
// the serial chain).  One extra workgroup of
// a step's launch updates the next diagonal block privately and factors it: one wave finds
// R22 R22^T = A22, all four then form U22 = R22^-1 by recursive doubling and
// M = U22^T U22, so the serial chain of small factorizations overlaps the bulk updates (at a
// super-block's first block the next diagonal block waits for the deferred update instead).
// Only the diagonal blocks of U are formed.  GPTQ's feedback into block J needs
// U[<J, J] = -U[<J,<J] R[<J, J] U_JJ only through E[:, <J] U[<J, J], and
// E[:, <J] U[<J,<J] = (W - Qhat)[:, <J] (the rounding error so far, in the layer's own
// basis), so the factor kept for block J is P[<J, J] = R[<J, J] U_JJ: for 64-column blocks
// exactly Z; for 128-column blocks [Z_a, Z_b - Z_a Z_b[a rows]], the second half coupled
// through U_ab = -U_a Z_b[a rows].
#include "device_util.h"
#include "kq_internal.h"

#include <algorithm>

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
// R).  Column j: p = A'_jj, R_jj = sqrt(p), R_lj = A'_lj / R_jj, and A'_lk -= R_lj R_kj for
// k < j.  The columns go in panels of 16 from the end: inside a panel the rank-1 updates
// touch only the panel's columns (A'_kj from lane k with v_readlane, so no LDS round trip per
// column), and after the panel the columns left of it take the panel's rank-16 update at once,
// A'[<16p, <16p] -= R[<16p, P] R[<16p, P]^T, as v_mfma_f32_16x16x4f32 products through LDS
// (Ab, read into registers first, is the scratch).  The same updates as column by column,
// in another order.  Rl's entries below the diagonal are left undefined.  Sets *flag on a
// non-positive pivot (the damped blocks' pivots are far from the denormal range, so the
// hardware reciprocal square root is used as it is).
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ void leaf_factor(float* Ab, float* Rl, float* rsq, int* flag) {
  const int l = threadIdx.x & 63;
  const int r16 = l & 15, k4 = l >> 4;
  float a[64];
#pragma unroll
  for (int k = 0; k < 64; k += 4) {
    const float4 v = *(const float4*)(Ab + l * LB + k);
    a[k] = v.x; a[k + 1] = v.y; a[k + 2] = v.z; a[k + 3] = v.w;
  }
  wave_sync();
  bool bad = false;
  float rs_own = 1.0f;   // 1 / R_ll, stored by lane l at the end
#pragma unroll
  for (int p = 3; p >= 0; --p) {
    const int lo = 16 * p;
#pragma unroll
    for (int j = lo + 15; j >= lo; --j) {
      // column j's entries in the panel's rows (uniform values), all read before they are
      // used so that the reads go back to back into distinct scalar registers
      float ck[16];
#pragma unroll
      for (int k = lo; k <= j; ++k) ck[k - lo] = lane_value(a[j], k);
      const float pj = ck[j - lo];
      const float rs = __builtin_amdgcn_rsqf(pj);
      const float f = a[j] * (rs * rs);
#pragma unroll
      for (int k = j - 1; k >= lo; --k) a[k] = fmaf(-f, ck[k - lo], a[k]);
      a[j] *= rs;
      Rl[l * LB + j] = a[j];
      rs_own = l == j ? rs : rs_own;
      bad |= (l == j) & !(pj > 0.0f);
    }
    if (p > 0) {
      wave_sync();
      // delta = R[<lo, P] R[<lo, P]^T, 16 x 16 tiles (lt, kt) on and above the diagonal
#pragma unroll
      for (int lt = 0; lt < p; ++lt)
#pragma unroll
        for (int kt = lt; kt < p; ++kt) {
          f32x4 acc = f32x4{};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Rl[(16 * lt + r16) * LB + lo + 4 * s + k4],
                                                       Rl[(16 * kt + r16) * LB + lo + 4 * s + k4],
                                                       acc, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) Ab[(16 * lt + 4 * k4 + i) * LB + 16 * kt + r16] = acc[i];
        }
      wave_sync();
      // row l, columns k < lo (those below the diagonal, never computed, are never read)
#pragma unroll
      for (int k = 0; k < lo; k += 4) {
        const float4 d = *(const float4*)(Ab + l * LB + k);
        a[k] -= d.x; a[k + 1] -= d.y; a[k + 2] -= d.z; a[k + 3] -= d.w;
      }
      wave_sync();
    }
  }
  rsq[l] = rs_own;
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
  {
    // diagonal block w: lane group 0 forms column c of its inverse (U_ic = (delta_ic -
    // sum_{k > i} R_ik U_kc) / R_ii, from the bottom up); groups 1..3 clear the blocks below
    const int b = 16 * w, c = r16;
    float rr[16][16], rq[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int k = 0; k < 16; k += 4) {
        const float4 v = *(const float4*)(Rl + (b + i) * LB + b + k);
        rr[i][k] = v.x; rr[i][k + 1] = v.y; rr[i][k + 2] = v.z; rr[i][k + 3] = v.w;
      }
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
      const float4 v = *(const float4*)(rsq + b + k);
      rq[k] = v.x; rq[k + 1] = v.y; rq[k + 2] = v.z; rq[k + 3] = v.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    float x[16];
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      float sum = 0.0f;
#pragma unroll
      for (int k = i + 1; k < 16; ++k) sum = fmaf(rr[i][k], x[k], sum);
      x[i] = i == c ? rq[i] : (i < c ? -rq[i] * sum : 0.0f);
    }
    if (k4 == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Ul[(b + i) * LB + b + c] = x[i];
    } else if (w + k4 <= 3) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Ul[(b + 16 * k4 + i) * LB + b + c] = 0.0f;
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

// Swizzled slabs of 64 columns in LDS (no padding).  Element (r, k) of a slab read by the MFMA
// with lanes along r (32 rows at one k; the other half wave at k + 1) sits at
// r * 64 + (k ^ (2 r & 62)), which puts the 64 lanes on 64 distinct banks.
__device__ __forceinline__ int sw(int r, int k) { return r * 64 + (k ^ ((2 * r) & 62)); }
// A 64 x 64 matrix read with lanes along columns (B operand): odd rows shifted by 32 columns.
__device__ __forceinline__ int swb(int k, int c) { return k * 64 + (c ^ ((k & 1) << 5)); }

// LDS for a leaf: X (64 x LB: A', the factor's scratch, then U) and Y (64 x LB for R, 64 for
// 1 / R_jj, 32 x LB scratch).
constexpr int LEAF_Y = 64 * LB + 64 + 32 * LB;

// Factor + invert the diagonal block held in X.  Writes U = R^-1 to Uout and
// M = U^T U = A'^-1 to Mout (64 x 64 row-major each).  Every thread of the 256-thread
// workgroup calls it.
__device__ __forceinline__ void leaf(float* X, float* Y, float* __restrict__ Uout,
                                     float* __restrict__ Mout, int* flag) {
  float* Rl = Y;
  float* rsq = Y + 64 * LB;
  float* Ts = rsq + 64;
  if (threadIdx.x < 64) leaf_factor(X, Rl, rsq, flag);
  __syncthreads();
  leaf_inverse(Rl, rsq, X, Ts);
  // M = U^T U.  U is upper, so quadrant (I, J) of 32 x 32 sums only k < 32 max(I, J) + 32:
  // wave 0 forms M00 and wave 1 M01 (= M10^T) over k < 32; waves 2 and 3 form the k < 32
  // and k >= 32 parts of M11.  M goes to LDS over R (no longer needed), then out with U.
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  const int ci = w >= 2 ? 32 : 0, cj = w == 0 ? 0 : 32, kb = w == 3 ? 32 : 0;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int k = 0; k < 32; k += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(X[(kb + k + kh) * LB + ci + l32],
                                               X[(kb + k + kh) * LB + cj + l32], acc, 0, 0, 0);
  float* Ml = Rl;
  if (w != 2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
      Ml[(ci + row) * LB + cj + l32] = acc[r];
      if (w == 1) Ml[(cj + l32) * LB + ci + row] = acc[r];
    }
  }
  __syncthreads();
  if (w == 2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float* m = Ml + (32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * LB + 32 + l32;
      *m = *m + acc[r];
    }
  }
  __syncthreads();
  for (int q = t; q < 64 * 16; q += 256) {
    const int r = q >> 4, c4 = (q & 15) * 4;
    *(float4*)(Uout + r * 64 + c4) = *(const float4*)(X + r * LB + c4);
    *(float4*)(Mout + r * 64 + c4) = *(const float4*)(Ml + r * LB + c4);
  }
}

// The last diagonal block [s0, s0 + 64), factored on its own.
__global__ __launch_bounds__(256) void leaf_kernel(const float* __restrict__ F, int64_t n,
                                                   int64_t s0, float* __restrict__ Uout,
                                                   float* __restrict__ Mout,
                                                   int* __restrict__ flag) {
  __shared__ __attribute__((aligned(16))) float X[64 * LB];
  __shared__ __attribute__((aligned(16))) float Y[LEAF_Y];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (threadIdx.x >> 4) + 16 * it, c4 = (threadIdx.x & 15) * 4;
    *(float4*)(X + r * LB + c4) = *(const float4*)(F + (s0 + r) * n + s0 + c4);
  }
  __syncthreads();
  leaf(X, Y, Uout, Mout, flag);
}

// Z = A12[I] M for one 128-row block: As (LDS, 128 x 64, sw layout) holds A12[I] on entry and
// Z on return; wave w forms rows 32 w .. 32 w + 31, all 64 columns.  Every thread calls it.
__device__ __forceinline__ void panel_z(float* As, const float* Ms) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l32 = lane & 31, kh = lane >> 5;
  f32x16 az[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float av[16], bv[16][2];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 32 * hh + 2 * kk + kh;
      av[kk] = As[sw(32 * w + l32, k)];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[kk][j] = Ms[swb(k, 32 * j + l32)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        az[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk], bv[kk][j], az[j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) As[sw(32 * w + 8 * (r >> 2) + 4 * kh + (r & 3), 32 * j + l32)] = az[j][r];
  __syncthreads();
}

// Z^T of rows i0 .. i0 + 128 (those below s0) into the free lower triangle:
// F[s0 + c][i0 + i] = Z[i][c], Z in As.
__device__ __forceinline__ void store_zt(float* __restrict__ F, int64_t n, int64_t s0, int64_t i0,
                                         const float* As) {
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rz = rsrc(F + s0 * n + i0);
  const int i = t & 127;
#pragma unroll
  for (int it = 0; it < 32; ++it) {
    const int c = 2 * it + (t >> 7);
    bstore(As[sw(i, c)], rz, i0 + i < s0 ? (c * (int)n + i) * 4 : OOB);
  }
}

// Step of the reverse factorization at block [s0, s0 + 64).  With A12 = F[0:s0, s0:s0+64]
// (the current Schur complement's column block) and M = A22^-1 = U22^T U22 from the previous
// step's leaf, the block's panel factor is Z = A12 M (= R12 U22 with R12 = A12 U22^T), and
// the trailing update is A11 -= A12 M A12^T = Z A12^T.  Z is GPTQ's feedback factor P for
// this 64-column block; it is stored transposed in the free lower triangle,
// F[s0 + c][r] = Z[r][c].  Workgroups, in order:
//   - with_leaf: workgroup 0 forms the next diagonal block D = [s0-64, s0)^2 privately,
//     D - Z_D A12[D]^T, and factors it (leaf), so the next step's factorization overlaps
//     the bulk update;
//   - zblocks "panel-factor" workgroups: Z for the 128-row blocks of rows [0, 128 zblocks)
//     (above the super-block), stored as Z^T;
//   - the tiles (upper 128 x 128 of [0, s0)^2) of the columns [pcol0, s0) that this step
//     updates now: Z for the tile's rows (A12[I] M), then C -= Z[I] A12[K]^T; the diagonal
//     tiles also store Z^T of their rows.  D is left to workgroup 0.
// 4 waves of v_mfma_f32_32x32x2f32; K = 64 in one LDS stage.  80 KB of LDS and at most 256
// registers per lane let two workgroups share a CU, so one tile's loads overlap another's
// products.
__global__ __launch_bounds__(256, 2) void update_kernel(float* __restrict__ F, int64_t n, int64_t s0,
                                                     const float* __restrict__ Mcur,
                                                     float* __restrict__ Unext,
                                                     float* __restrict__ Mnext,
                                                     int* __restrict__ flag, int64_t pcol0,
                                                     int zblocks, int with_leaf) {
  __shared__ __attribute__((aligned(16))) float As[128 * 64];
  __shared__ __attribute__((aligned(16))) float Bs[128 * 64];
  __shared__ __attribute__((aligned(16))) float Ms[64 * 64];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, l32 = lane & 31, kh = lane >> 5;
  const int64_t d0 = s0 - 64;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int q = t + 256 * it, r = q >> 4, c4 = (q & 15) * 4;
    const float4 v = *(const float4*)(Mcur + r * 64 + c4);
    Ms[swb(r, c4)] = v.x; Ms[swb(r, c4 + 1)] = v.y; Ms[swb(r, c4 + 2)] = v.z; Ms[swb(r, c4 + 3)] = v.w;
  }
  int b = blockIdx.x;
  if (with_leaf && b == 0) {
    // A12[D] -> As rows 0..63, D -> Bs as the leaf's X (row stride LB)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = t + 256 * it, r = q >> 4, c4 = (q & 15) * 4;
      const float4 v = *(const float4*)(F + (d0 + r) * n + s0 + c4);
      As[sw(r, c4)] = v.x; As[sw(r, c4 + 1)] = v.y; As[sw(r, c4 + 2)] = v.z; As[sw(r, c4 + 3)] = v.w;
      *(float4*)(Bs + r * LB + c4) = *(const float4*)(F + (d0 + r) * n + d0 + c4);
    }
    const int wi = w >> 1, wj = w & 1;
    __syncthreads();
    // Z_D = A12[D] M into As rows 64..127
    f32x16 acc = f32x16{};
#pragma unroll 8
    for (int k = 0; k < 64; k += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[sw(32 * wi + l32, k + kh)],
                                                 Ms[swb(k + kh, 32 * wj + l32)], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) As[sw(64 + 32 * wi + 8 * (r >> 2) + 4 * kh + (r & 3), 32 * wj + l32)] = acc[r];
    __syncthreads();
    // D' = D - Z_D A12[D]^T
    f32x16 acc2 = f32x16{};
#pragma unroll 8
    for (int k = 0; k < 64; k += 2)
      acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(As[sw(64 + 32 * wi + l32, k + kh)],
                                                  As[sw(32 * wj + l32, k + kh)], acc2, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float* d = Bs + (32 * wi + 8 * (r >> 2) + 4 * kh + (r & 3)) * LB + 32 * wj + l32;
      *d = *d - acc2[r];
    }
    __syncthreads();
    leaf(Bs, As, Unext, Mnext, flag);
    return;
  }
  if (with_leaf) b -= 1;
  if (b < zblocks) {
    // panel factor of rows i0 .. i0 + 127 (all below s0): Z = A12[I] M, stored as Z^T
    const int64_t i0 = (int64_t)b * 128;
    const __amdgpu_buffer_rsrc_t ra = rsrc(F + i0 * n + s0);
    float4 va[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = (t >> 4) + 16 * it, off = (r * (int)n + (t & 15) * 4) * 4;
      va[it] = bload4(ra, i0 + r < s0 ? off : OOB);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = (t >> 4) + 16 * it, c4 = (t & 15) * 4;
      As[sw(r, c4)] = va[it].x; As[sw(r, c4 + 1)] = va[it].y; As[sw(r, c4 + 2)] = va[it].z; As[sw(r, c4 + 3)] = va[it].w;
    }
    __syncthreads();
    panel_z(As, Ms);
    store_zt(F, n, s0, i0, As);
    return;
  }
  b -= zblocks;
  // tile (tm, tn), tm <= tn, of the columns tn >= pcol0 / 128, enumerated column by column
  int tn = (int)(pcol0 / 128), tm = b;
  while (tm > tn) { tm -= tn + 1; ++tn; }
  const int64_t i0 = (int64_t)tm * 128, j0 = (int64_t)tn * 128;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  // this lane's tile entries: rows rbase + 32 i + 8 (r / 4) + r % 4, columns cbase + 32 j
  const int64_t rbase = i0 + wm + 4 * kh, cbase = j0 + wn + l32;
  const int rlim = (int)min((int64_t)128, s0 - rbase), clim = (int)min((int64_t)128, s0 - cbase);
  // A12[I] and A12[K] (rows past s0 read as 0): all loads first
  const __amdgpu_buffer_rsrc_t ra = rsrc(F + i0 * n + s0);
  const __amdgpu_buffer_rsrc_t rb = rsrc(F + j0 * n + s0);
  float4 va[8], vb[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = (t >> 4) + 16 * it, off = (r * (int)n + (t & 15) * 4) * 4;
    va[it] = bload4(ra, i0 + r < s0 ? off : OOB);
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = (t >> 4) + 16 * it, off = (r * (int)n + (t & 15) * 4) * 4;
    vb[it] = bload4(rb, j0 + r < s0 ? off : OOB);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = (t >> 4) + 16 * it, c4 = (t & 15) * 4;
    As[sw(r, c4)] = va[it].x; As[sw(r, c4 + 1)] = va[it].y; As[sw(r, c4 + 2)] = va[it].z; As[sw(r, c4 + 3)] = va[it].w;
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = (t >> 4) + 16 * it, c4 = (t & 15) * 4;
    Bs[sw(r, c4)] = vb[it].x; Bs[sw(r, c4 + 1)] = vb[it].y; Bs[sw(r, c4 + 2)] = vb[it].z; Bs[sw(r, c4 + 3)] = vb[it].w;
  }
  __syncthreads();
  // Z[I] = A12[I] M
  panel_z(As, Ms);
  // the diagonal tiles also store Z^T
  if (tm == tn) store_zt(F, n, s0, i0, As);
  // C -= Z[I] A12[K]^T in two halves of 32 k; each half's operands are read before its MFMAs
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float av[16][2], bv[16][2];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 32 * hh + 2 * kk + kh;
#pragma unroll
      for (int i = 0; i < 2; ++i) av[kk][i] = As[sw(wm + 32 * i + l32, k)];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[kk][j] = Bs[sw(wn + 32 * j + l32, k)];
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
  // the tile's old values: all loads first, then all stores.  This lane's entries sit at tile
  // rows wm + 4 kh + 32 i + 8 (r / 4) + r % 4 and columns wn + l32 + 32 j; entries past s0 or
  // inside the next diagonal block D (which workgroup 0 owns) are masked.
  const __amdgpu_buffer_rsrc_t rc = rsrc(F + i0 * n + j0);
  int off[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ro = 32 * i + 8 * (r >> 2) + (r & 3);
        const bool in_d = rbase + ro >= d0 && cbase + 32 * j >= d0;
        off[i][j][r] = (ro < rlim && 32 * j < clim && !in_d)
                           ? ((wm + 4 * kh + ro) * (int)n + wn + l32 + 32 * j) * 4
                           : OOB;
      }
  float cv[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) cv[i][j][r] = bload(rc, off[i][j][r]);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) bstore(cv[i][j][r] - acc[i][j][r], rc, off[i][j][r]);
}

// Moves each diagonal block's U_JJ from the block buffer into place.
__global__ void finalize_kernel(float* __restrict__ F, int64_t n, const float* __restrict__ Ubuf) {
  const int64_t b = blockIdx.x;
  for (int q = threadIdx.x; q < 64 * 64; q += 256)
    F[(64 * b + (q >> 6)) * n + 64 * b + (q & 63)] = Ubuf[b * 4096 + q];
}

// For GPTQ blocks of 128 columns, the 128 x 128 diagonal block of U = R^-1 from its two
// 64-blocks a, b: U_ab = -U_a R_ab U_b = -U_a Z_b[a rows] (Z_b^T lies in the lower triangle).
// One workgroup per 128-block; each wave forms a 32 x 32 quadrant (v_mfma_f32_32x32x2f32).
__global__ __launch_bounds__(256) void ujj128_kernel(float* __restrict__ F, int64_t n) {
  __shared__ float Ua[64 * LP];
  __shared__ float Zs[64 * LP];
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  const int64_t a0 = (int64_t)blockIdx.x * 128, b0 = a0 + 64;
  for (int q = t; q < 64 * 64; q += 256) {
    const int r = q >> 6, c = q & 63;
    Ua[r * LP + c] = F[(a0 + r) * n + a0 + c];
    Zs[c * LP + r] = F[(b0 + r) * n + a0 + c];   // Z_b[a0 + c][r] stored at F[b0 + r][a0 + c]
  }
  __syncthreads();
  const int wi = w >> 1, wj = w & 1;
  f32x16 acc = f32x16{};
#pragma unroll 8
  for (int k = 0; k < 64; k += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ua[(32 * wi + l32) * LP + k + kh],
                                               Zs[(k + kh) * LP + 32 * wj + l32], acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    F[(a0 + 32 * wi + 8 * (r >> 2) + 4 * kh + (r & 3)) * n + b0 + 32 * wj + l32] = -acc[r];
}

// GPTQ feedback factors P[<J, J] above each B x B diagonal block, from the Z^T of the
// factorization (lower triangle).  B = 64: P = Z.  B = 128 (blocks a, b):
// P = [Z_a, Z_b - Z_a Z_b[a rows]].  One workgroup per (128-row tile, block J) with the tile
// above the block; 4 waves of v_mfma_f32_32x32x2f32 for the B = 128 correction.
template <int B>
__global__ __launch_bounds__(256) void pmat_kernel(float* __restrict__ F, int64_t n) {
  __shared__ float Za[128 * LP];
  __shared__ float Zb[B == 128 ? 128 * LP : 4];
  __shared__ float Zba[B == 128 ? 64 * LP : 4];
  int idx = blockIdx.x, J = 1;
  // tiles of 128 rows above block J: ceil(J * B / 128)
  for (;;) {
    const int nt = (J * B + 127) / 128;
    if (idx < nt) break;
    idx -= nt;
    ++J;
  }
  const int64_t r0 = (int64_t)idx * 128, a0 = (int64_t)J * B, rows = min((int64_t)128, a0 - r0);
  const int t = threadIdx.x;
  // lanes along r: coalesced reads of Z^T rows.  Batches of loads are issued before any is
  // used: rows past `rows` are read at the last row and stored as zero (a select, not a
  // branch around the load, which would make every load wait for the ones before it).
  constexpr int NQ = 64 * 128 / 256;
#pragma unroll
  for (int q0 = 0; q0 < NQ; q0 += 8) {
    float va[8], vb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = t + 256 * (q0 + i), c = q >> 7, r = q & 127;
      const int64_t rr = r0 + min(r, (int)rows - 1);
      va[i] = F[(a0 + c) * n + rr];
      if constexpr (B == 128) vb[i] = F[(a0 + 64 + c) * n + rr];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = t + 256 * (q0 + i), c = q >> 7, r = q & 127;
      Za[r * LP + c] = r < rows ? va[i] : 0.0f;
      if constexpr (B == 128) Zb[r * LP + c] = r < rows ? vb[i] : 0.0f;
    }
  }
  if constexpr (B == 128) {
    float vz[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = t + 256 * i, c = q >> 6, r = q & 63;
      vz[i] = F[(a0 + 64 + c) * n + a0 + r];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = t + 256 * i, c = q >> 6, r = q & 63;
      Zba[r * LP + c] = vz[i];
    }
  }
  __syncthreads();
  for (int q = t; q < 128 * 64; q += 256) {
    const int r = q >> 6, c = q & 63;
    if (r < rows) F[(r0 + r) * n + a0 + c] = Za[r * LP + c];
  }
  if constexpr (B == 128) {
    const int w = t >> 6, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll 4
    for (int k = 0; k < 64; k += 2) {
      const float av = Za[(32 * w + l32) * LP + k + kh];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, Zba[(k + kh) * LP + 32 * j + l32], acc[j],
                                                      0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * w + 8 * (r >> 2) + 4 * kh + (r & 3), c = 32 * j + l32;
        if (row < rows) F[(r0 + row) * n + a0 + 64 + c] = Zb[row * LP + c] - acc[j][r];
      }
  }
}

}  // namespace

// Copies HX into the workspace matrix F, damps it and factors it (H_d = R R^T).  On return F
// holds, above its B x B diagonal blocks, GPTQ's feedback factors P = R[<J, J] U_JJ, and in
// the upper triangles of those blocks U_JJ (U = R^-1 = chol_upper(H_d^-1)); the strictly
// lower triangle keeps the factorization's panels Z^T (not part of U or P).
// T is scratch of 128 n floats.
kq_status damp_and_factor(const float* HX, float* F, float* T, uint8_t* dead, double* lam,
                          int* flag, int64_t n, float damp, int B, hipStream_t s) {
  if (n % NB != 0) return fail(KQ_ESHAPE, "factorization needs n %% %d == 0", NB);
  if ((B != 64 && B != 128) || n % B != 0) return fail(KQ_ESHAPE, "bad GPTQ block %d", B);
  // HX == NULL: F already holds the matrix
  if (HX) KQ_HIP(hipMemcpyAsync(F, HX, n * n * sizeof(float), hipMemcpyDeviceToDevice, s));
  damp_stats_kernel<<<1, 1024, 0, s>>>(F, n, dead, damp, lam);
  KQ_LAUNCHED("damp_stats_kernel");
  add_diag_kernel<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s>>>(F, n, lam);
  KQ_LAUNCHED("add_diag_kernel");
  // reverse Cholesky.  The diagonal blocks' U_JJ = R_JJ^-1 and M_JJ = U_JJ^T U_JJ are kept
  // in the block buffers T (64 n floats each); F holds A above the diagonal blocks and the
  // panel factors Z^T below them.
  float* Ubuf = T;
  float* Mbuf = T + 64 * n;
  const int64_t nb = n / NB;
  leaf_kernel<<<1, 256, 0, s>>>(F, n, n - NB, Ubuf + (nb - 1) * 4096, Mbuf + (nb - 1) * 4096, flag);
  KQ_LAUNCHED("leaf_kernel");
  // super-blocks of SB columns (a multiple of 128, aligned to column 0): a step updates the
  // columns of its own super-block that are still to come; the columns left of it take the
  // super-block's whole update at its first block.  Worth it once the matrix outgrows the
  // last-level cache: measured for the quantize stage (factor + GPTQ, out = 4096), 4096 wide
  // 2.41 ms with no deferral against 2.66 ms at SB = 512; 8192 wide 7.80 ms at 1024 against
  // 8.89 ms with none; 11008 wide 13.83 ms at 1024, 14.24 at 512, 17.55 with none.  (Tests
  // can pick other widths: the same updates, summed in another order.)
  const int64_t n128 = ceil_div(n, 128) * 128;
  int64_t SB = testing_value(KQ_TESTING_FACTOR_SUPERBLOCK,
                             n * n * (int64_t)sizeof(float) > ((int64_t)128 << 20) ? 1024 : n128);
  if (SB < 128 || SB % 128 != 0) SB = 1024;
  for (int64_t s0 = n - NB; s0 >= NB; s0 -= NB) {
    const int64_t jb = s0 / NB;
    const int64_t S0 = (s0 / SB) * SB;          // first column of this block's super-block
    const bool first = s0 == S0;                 // the super-block's first (leftmost) block
    const int64_t m = ceil_div(s0, 128);
    int64_t ptiles = 0;
    if (!first)
      for (int64_t tn = S0 / 128; tn < m; ++tn) ptiles += tn + 1;
    // Z^T for the rows above the super-block (at its first block: for every row above s0)
    const int64_t zb = first ? m : S0 / 128;
    const int64_t grid = (first ? 0 : 1) + zb + ptiles;
    update_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(
        F, n, s0, Mbuf + jb * 4096, Ubuf + (jb - 1) * 4096, Mbuf + (jb - 1) * 4096, flag, S0,
        (int)zb, first ? 0 : 1);
    KQ_LAUNCHED("update_kernel");
    if (first) {
      // F[0:S0, 0:S0] (upper tiles) -= A12 Z^T over the super-block's columns [S0, S0 + K):
      // A12 = F[0:S0, S0:S0+K], Z^T = F[S0:S0+K, 0:S0] (the lower triangle)
      GemmArgs g{};
      g.M = S0; g.N = S0; g.K = std::min<int64_t>(SB, n - S0);
      g.A = F + S0; g.lda = n; g.transA = false;
      g.B = F + S0 * n; g.ldb = n; g.transB = false;
      g.C = F; g.ldc = n; g.alpha = -1.0f; g.accumulate = true; g.upper_only = true;
      g.split_k = 1; g.batch = 1;
      KQ_TRY(gemm_f32(g, s));
      leaf_kernel<<<1, 256, 0, s>>>(F, n, s0 - NB, Ubuf + (jb - 1) * 4096, Mbuf + (jb - 1) * 4096,
                                    flag);
      KQ_LAUNCHED("leaf_kernel");
    }
  }
  finalize_kernel<<<dim3((unsigned)nb), dim3(256), 0, s>>>(F, n, Ubuf);
  KQ_LAUNCHED("finalize_kernel");
  // GPTQ's feedback factors: the B x B diagonal blocks of U and P[<J, J] = R[<J, J] U_JJ
  if (B == 128) {
    ujj128_kernel<<<dim3((unsigned)(n / 128)), dim3(256), 0, s>>>(F, n);
    KQ_LAUNCHED("ujj128_kernel");
  }
  int64_t ptiles = 0;
  for (int64_t J = 1; J < n / B; ++J) ptiles += ceil_div(J * B, 128);
  if (ptiles > 0) {
    if (B == 128) pmat_kernel<128><<<dim3((unsigned)ptiles), dim3(256), 0, s>>>(F, n);
    else pmat_kernel<64><<<dim3((unsigned)ptiles), dim3(256), 0, s>>>(F, n);
    KQ_LAUNCHED("pmat_kernel");
  }
  return KQ_OK;
}

}  // namespace kq
