// FlipFlop Hessian factors: A = E[(g^T B^-1 g) x x^T] / m and B = E[(x^T A^-1 x) g g^T] / n,
// by the alternating fixed-point iteration from B = I.
//
// WaterKron and FlipFlop Hessian, Table 1 (row "FlipFlop") and its caption (the alternating
// fixed-point iteration from the identity); the 1/m and 1/n are the classical flip-flop's
// (the maximum-likelihood fit of a Kronecker covariance to the samples vec(x g^T)), which
// A (x) B does not depend on.  E is the mean over the T calibration tokens.
//
// One half step, A from B (the other half swaps the streams):
//   1. B = R R^T (the engine's reverse Cholesky, no damping; a zero diagonal counts as 1),
//      then the explicit U = R^-1 (upper): its diagonal blocks and the panels P = R U_JJ
//      come from the factorization, the blocks above from U[<J, J] = -U[<J,<J] P[<J, J],
//      one fp32 MFMA product per block column.  g^T B^-1 g = |U g|^2.
//   2. w_t = |U g_t|^2 for every token: bf16 MFMA products of the stream with U, fp32
//      accumulation, the squares summed per token in the epilogue; tiles left of the
//      diagonal of U are skipped.  U enters as two bf16 terms, U_hi = bf16(U) and
//      U_lo = bf16(U - U_hi), multiplied into the same accumulators (the contraction runs
//      twice), so U carries about 16 significant bits: with U_hi alone its rounding is the
//      same in every token and its error in the factors does not average out.
//   3. A = sum_t a_t x_t^T with a_t = (w_t / (T m)) x_t: the weight goes on one side only,
//      so the other operand is the exact bf16 stream x.  a enters as two bf16 terms,
//      a_hi = bf16(a) and a_lo = bf16(a - a_hi) (about 16 significant bits; with a rounded
//      once the per-token weights' rounding would not average out, a few heavy tokens
//      dominating the sum), through the SYRK's kernel with a second stream for the column
//      channels: the lower tiles of a_hi x^T, then of a_lo x^T added to them, then the lower
//      triangle mirrored, so A is exactly symmetric.  Two products of width n, half the
//      work of a SYRK of the stream [y_hi y_lo] of width 2n.
//
// qform_kernel: 256-token x 256-output tiles, 4 waves of 128 x 128 (4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16); stages of 32 contraction indices: both panels (256 rows x 64
// bytes each) copied into LDS by the load unit (global_load_lds, 16 bytes per lane) in a
// ring of four stages, operands read with ds_read_b128 (8 consecutive contraction indices of
// one row per lane, as the MFMA takes them); the 16-byte chunks of row r sit in slot
// c ^ ((r >> 2) & 3), which spreads the rows read together over the banks.
#include "device_util.h"
#include "kq_internal.h"

#include <math.h>

#include <algorithm>
#include <vector>

namespace kq {

kq_status damp_and_factor(const float* HX, float* F, float* T, uint8_t* dead, double* lam,
                          int* flag, int64_t n, float damp, int B, hipStream_t s);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int QT = 256;                 // tile edge (tokens, outputs)
constexpr int QK = 32;                  // contraction indices per stage
constexpr int QPANEL = QT * QK;         // bf16 elements of one panel (16 KB)
constexpr int QSTAGE = 2 * QPANEL;      // both panels of a stage (32 KB)
constexpr int QNST = 4;                 // stages in the ring (128 KB)
constexpr int QCOPIES = QPANEL * 2 / 1024 / 4;   // 1 KB wave copies per panel and wave (4)

__device__ __forceinline__ unsigned short bf16_rne(float x) {
  unsigned u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// Sixteen zero bytes: the source of every copy lane whose row lies outside the matrix, so that
// each wave issues the same number of copies per stage and the vmcnt waits stay exact.
__device__ __attribute__((aligned(16))) uint32_t q_zero_chunk[4];

__device__ __forceinline__ int qswz(int r) { return (r >> 2) & 3; }

struct QArgs {
  const uint16_t* S;   // stream, T x k bf16, leading dim lds (elements)
  int64_t lds;
  const uint16_t* U;   // k x k bf16, upper triangular (row j: U[j, j..k)), leading dim k
  int64_t ulo;         // offset (elements) from U to the k x k low part U_lo
  int64_t T;
  int k;
  float* part;         // T x np partial sums of squares (np = 2 * ceil(k / 256))
  int np;
  int ntt, njt;        // token tiles, output tiles
  int ntt_x;           // token tiles per XCD
  int per_xcd;         // tiles per XCD: ntt_x * njt
};

constexpr int QBAND = 8;                // token tiles per band of an XCD's walk

// part[t, 2 jt + wc] = sum over the 128 outputs j of wave column wc of tile jt of
// (sum_i U[j, i] S[t, i])^2.
// Stage s of the ring: the operands of its first 16 contraction indices are in registers
// (xa, xb); the second 16 (ya, yb) are read while the first are multiplied; then, once this
// wave's copies of stage s+1 have landed and every wave's reads of stage s are done (one
// barrier), stage s's buffer is refilled with stage s + QNST and the first operands of stage
// s+1 are read while the second half of stage s is multiplied.  Each buffer is its own LDS
// object, so the compiler can tell the reads of one stage from the copies into another.
__global__ __launch_bounds__(256) void qform_kernel(QArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t b0[QSTAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[QSTAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t b2[QSTAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t b3[QSTAGE];
  // workgroup u runs on XCD u mod 8; each XCD takes its own range of ntt_x token tiles, in
  // bands of QBAND token tiles walked output tile by output tile, so the 32 tiles an XCD
  // runs at once span 8 token panels and 4 panels of U (rather than 2 and 16) and share
  // their stage windows in its L2
  const int u = blockIdx.x;
  const int l = u >> 3;
  const int band = l / (QBAND * a.njt);
  const int tb0 = band * QBAND;
  const int bt = min(QBAND, a.ntt_x - tb0);
  if (bt <= 0) return;
  const int w = l - band * QBAND * a.njt;
  const int jt = w / bt;
  const int tt = (u & 7) * a.ntt_x + tb0 + w % bt;
  if (tt >= a.ntt || jt >= a.njt) return;
  const int64_t t0 = (int64_t)tt * QT;
  const int j0 = jt * QT;
  const int i_begin = j0;                       // U[j, i] = 0 for i < j
  const int nst = (a.k - i_begin) / QK;         // k % 128 == 0; stages per pass over U
  // stages 0 .. nst - 1 multiply by U_hi, nst .. 2 nst - 1 by U_lo (the same stream columns)
  const int nst_round = (2 * nst + QNST - 1) / QNST * QNST;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  // copy sources: wave w fills 1 KB blocks 4w + c of each panel (16 rows of 64 bytes); lane l
  // writes slot l & 3 of row 16 (4w + c) + (l >> 2), which holds chunk (l & 3) ^ qswz(row)
  const uint16_t* zero = (const uint16_t*)q_zero_chunk;
  const uint16_t* srcS[QCOPIES];
  const uint16_t* srcU[QCOPIES];
#pragma unroll
  for (int c = 0; c < QCOPIES; ++c) {
    const int row = 16 * (4 * wave + c) + (lane >> 2);
    const int chunk = (lane & 3) ^ qswz(row);
    srcS[c] = t0 + row < a.T ? a.S + (t0 + row) * a.lds + i_begin + 8 * chunk : zero;
    srcU[c] = j0 + row < a.k ? a.U + (int64_t)(j0 + row) * a.k + i_begin + 8 * chunk : zero;
  }
  auto issue = [&](int s, uint16_t* buf) {
    const bool live = s < 2 * nst;
    const bool lo = s >= nst;
    const int sc = lo ? s - nst : s;
#pragma unroll
    for (int c = 0; c < QCOPIES; ++c) {
      const uint16_t* ps = live && srcS[c] != zero ? srcS[c] + sc * QK : zero;
      const uint16_t* pu = live && srcU[c] != zero ? srcU[c] + (lo ? a.ulo : 0) + sc * QK : zero;
      __builtin_amdgcn_global_load_lds((const void*)ps,
                                       (__attribute__((address_space(3))) void*)(buf + (4 * wave + c) * 512),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)pu,
                                       (__attribute__((address_space(3))) void*)(buf + QPANEL + (4 * wave + c) * 512),
                                       16, 0, 0);
    }
  };

  // operand read offsets (elements) inside a panel: row 32 b + (l & 31) of the wave's half,
  // chunk 2 h + (l >> 5)
  int offS[2][4], offU[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int rs = 128 * wr + 32 * b + (lane & 31), ru = 128 * wc + 32 * b + (lane & 31);
      const int c = 2 * h + (lane >> 5);
      offS[h][b] = rs * QK + 8 * (c ^ qswz(rs));
      offU[h][b] = QPANEL + ru * QK + 8 * (c ^ qswz(ru));
    }
  auto read = [&](const uint16_t* buf, int h, bf16x8 (&av)[4], bf16x8 (&bv)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      av[b] = *(const bf16x8*)(buf + offS[h][b]);
      bv[b] = *(const bf16x8*)(buf + offU[h][b]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x16{};
  auto mma = [&](const bf16x8 (&av)[4], const bf16x8 (&bv)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bv[n], acc[m][n], 0, 0, 0);
  };

  bf16x8 xa[4], xb[4], ya[4], yb[4];
  issue(0, b0);
  issue(1, b1);
  issue(2, b2);
  issue(3, b3);
  // this wave's copies of stage 0 have landed once at most those of stages 1..3 remain
  __builtin_amdgcn_s_waitcnt(wait_vm(2 * QCOPIES * (QNST - 1)));
  lds_barrier();
  read(b0, 0, xa, xb);
#define KQ_QF_STEP(J, CUR, NXT)                                    \
  {                                                                \
    read(CUR, 1, ya, yb);                                          \
    mma(xa, xb);                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           \
    }                                                              \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);             \
    __builtin_amdgcn_sched_barrier(0);                             \
    __builtin_amdgcn_s_waitcnt(wait_vm(2 * QCOPIES * (QNST - 2))); \
    __builtin_amdgcn_s_waitcnt(0xc07f);                            \
    lds_barrier();                                                 \
    issue(s0 + (J) + QNST, CUR);                                   \
    read(NXT, 0, xa, xb);                                          \
    mma(ya, yb);                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);           \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);           \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);           \
    }                                                              \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);             \
    __builtin_amdgcn_sched_barrier(0);                             \
  }
  for (int s0 = 0; s0 < nst_round; s0 += QNST) {
    KQ_QF_STEP(0, b0, b1)
    KQ_QF_STEP(1, b1, b2)
    KQ_QF_STEP(2, b2, b3)
    KQ_QF_STEP(3, b3, b0)
  }
#undef KQ_QF_STEP
  // the ring's trailing copies (zeros) must land, and every wave's last reads be done, before
  // the LDS is reused
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __builtin_amdgcn_s_waitcnt(0xc07f);
  lds_barrier();

  // epilogue: lane holds output column l & 31 of each 32 x 32 block, rows
  // 8 (r / 4) + 4 (l / 32) + r % 4.  Sum the squares over the wave's 128 columns: over the
  // four column blocks in registers, then over the 32 lanes of a half-wave through LDS.
  float* red = (float*)(wave == 0 ? b0 : wave == 1 ? b1 : wave == 2 ? b2 : b3);   // 128 x 33 floats
  const int l32 = lane & 31, rh = (lane >> 5) * 4;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) v = fmaf(acc[m][n][r], acc[m][n][r], v);
      const int row = 32 * m + 8 * (r >> 2) + rh + (r & 3);
      red[row * 33 + l32] = v;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = lane + 64 * h;
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) v += red[row * 33 + c];
    const int64_t t = t0 + 128 * wr + row;
    if (t < a.T) a.part[t * a.np + 2 * jt + wc] = v;
  }
}

// a = c * sum_p part[t, p] * S[t, :]: out[t, 0:k] = bf16(a) and out[t, k:2k] =
// bf16(a - bf16(a)) (round to nearest even; the remainder is exact in fp32); one workgroup per
// token, 8 channels per thread and step.
__global__ __launch_bounds__(256) void ff_scale_kernel(const uint16_t* __restrict__ S, int64_t lds,
                                                       int k, const float* __restrict__ part,
                                                       int np, float c, uint16_t* __restrict__ out,
                                                       int64_t ldo) {
  const int64_t t = blockIdx.x;
  __shared__ float sf;
  if (threadIdx.x < 64) {
    float w = 0.f;
    for (int p = threadIdx.x; p < np; p += 64) w += part[t * np + p];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o);
    if (threadIdx.x == 0) sf = c * w;
  }
  __syncthreads();
  const float f = sf;
  for (int i = 8 * threadIdx.x; i < k; i += 8 * 256) {
    const u32x4 v = *(const u32x4*)(S + t * lds + i);
    u32x4 oh, ol;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      unsigned rh = 0, rl = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x = __uint_as_float(((v[h] >> (16 * e)) & 0xffffu) << 16) * f;
        const unsigned hi = bf16_rne(x);
        const unsigned lo = bf16_rne(x - __uint_as_float(hi << 16));
        rh |= hi << (16 * e);
        rl |= lo << (16 * e);
      }
      oh[h] = rh;
      ol[h] = rl;
    }
    *(u32x4*)(out + t * ldo + i) = oh;
    *(u32x4*)(out + t * ldo + k + i) = ol;
  }
}

// The diagonal 128-blocks of U: the upper triangles of F's diagonal blocks (U_JJ); below
// the diagonal F holds the factorization's panels, which are not part of U.
__global__ __launch_bounds__(256) void copy_diag_blocks(const float* __restrict__ F,
                                                        float* __restrict__ U, int64_t k) {
  const int64_t J = blockIdx.x;
  for (int e = threadIdx.x; e < 128 * 128; e += 256) {
    const int r = e >> 7, c = e & 127;
    U[(J * 128 + r) * k + J * 128 + c] = c >= r ? F[(J * 128 + r) * k + J * 128 + c] : 0.0f;
  }
}

// Two-term bf16 copy of an fp32 matrix (round to nearest even): hi = bf16(v),
// lo = bf16(v - hi) (v - hi is exact in fp32), 4 entries per thread.
__global__ __launch_bounds__(256) void to_bf16_pair_kernel(const float* __restrict__ src,
                                                           uint16_t* __restrict__ hi,
                                                           uint16_t* __restrict__ lo,
                                                           int64_t count) {
  const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (i >= count) return;
  const float4 v = *(const float4*)(src + i);
  const float e[4] = {v.x, v.y, v.z, v.w};
  unsigned short oh[4], ol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    oh[j] = bf16_rne(e[j]);
    ol[j] = bf16_rne(e[j] - __uint_as_float((unsigned)oh[j] << 16));
  }
  *(ushort4*)(hi + i) = make_ushort4(oh[0], oh[1], oh[2], oh[3]);
  *(ushort4*)(lo + i) = make_ushort4(ol[0], ol[1], ol[2], ol[3]);
}

__global__ void identity_kernel(float* __restrict__ M, int64_t k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < k * k) M[i] = (i / k == i % k) ? 1.f : 0.f;
}

struct Workspace {
  uint16_t* Ss;    // weighted stream as two bf16 terms side by side, T x ldS (ldS >= 2 kmax)
  int64_t ldS;
  float* part;     // T x npmax
  float* F;        // factorization, kmax^2
  float* Tsc;      // factorization scratch, 128 kmax
  float* Uf;       // explicit inverse factor, kmax^2
  uint16_t* Ub;    // its two-term bf16 copy: U_hi (kmax^2), then U_lo (kmax^2)
  uint8_t* dead;   // kmax
  double* lam;
  int* flag;
};

inline int64_t al256(int64_t b) { return (b + 255) / 256 * 256; }

int64_t layout(int64_t T, int64_t n, int64_t m, char* base, Workspace* w) {
  const int64_t k = std::max(n, m);
  const int64_t np = 2 * ((k + 255) / 256);
  int64_t off = 0;
  auto take = [&](int64_t bytes) { const int64_t o = off; off += al256(bytes); return base ? base + o : nullptr; };
  Workspace x;
  x.ldS = (2 * k + 7) / 8 * 8;
  x.Ss = (uint16_t*)take(T * x.ldS * 2);
  x.part = (float*)take(T * np * 4);
  x.F = (float*)take(k * k * 4);
  x.Tsc = (float*)take(128 * k * 4);
  x.Uf = (float*)take(k * k * 4);
  x.Ub = (uint16_t*)take(2 * k * k * 2);
  x.dead = (uint8_t*)take(k);
  x.lam = (double*)take(8);
  x.flag = (int*)take(4);
  if (w) *w = x;
  return off;
}

// Ub = [bf16(U), bf16(U - bf16(U))] (k x k each), U = R^-1 for M = R R^T (no damping; zero
// diagonals count as 1).
kq_status inverse_factor(const float* M, int64_t k, const Workspace& w, hipStream_t s) {
  KQ_TRY(explicit_inverse_factor(M, k, 0.0f, w.F, w.Tsc, w.dead, w.lam, w.flag, w.Uf, s));
  const int64_t cnt = k * k;
  to_bf16_pair_kernel<<<dim3((unsigned)ceil_div(cnt / 4, 256)), dim3(256), 0, s>>>(w.Uf, w.Ub,
                                                                                  w.Ub + cnt, cnt);
  KQ_LAUNCHED("to_bf16_pair_kernel");
  return KQ_OK;
}

// part <- per-token partial sums of |U s_t|^2 (U = w.Ub, k x k)
kq_status quadratic_forms(const uint16_t* S, int64_t lds, int64_t T, int64_t k, const Workspace& w,
                          hipStream_t s) {
  QArgs a;
  a.S = S; a.lds = lds; a.U = w.Ub; a.ulo = k * k; a.T = T; a.k = (int)k; a.part = w.part;
  a.njt = (int)((k + QT - 1) / QT);
  a.np = 2 * a.njt;
  a.ntt = (int)((T + QT - 1) / QT);
  a.ntt_x = (int)ceil_div(a.ntt, 8);
  a.per_xcd = a.ntt_x * a.njt;
  const int64_t grid = 8 * (int64_t)a.per_xcd;
  if (grid > 0x7fffffff) return fail(KQ_ESHAPE, "kq_flipflop: too many tiles");
  qform_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  KQ_LAUNCHED("qform_kernel");
  return KQ_OK;
}

// HIP events around the phases of every half step (factor + inverse factor, quadratic
// forms, scaling, SYRK), on the call's stream; read once the stream has drained.
struct PhaseTimer {
  bool on = false;
  std::vector<hipEvent_t> ev;   // 5 per half step
  kq_status mark(hipStream_t s) {
    if (!on) return KQ_OK;
    hipEvent_t e;
    KQ_HIP(hipEventCreate(&e));
    ev.push_back(e);
    KQ_HIP(hipEventRecord(e, s));
    return KQ_OK;
  }
  kq_status read(double* ms) {
    for (int p = 0; p < 4; ++p) ms[p] = 0.0;
    for (size_t h = 0; h + 4 < ev.size(); h += 5)
      for (int p = 0; p < 4; ++p) {
        float t = 0.f;
        KQ_HIP(hipEventElapsedTime(&t, ev[h + p], ev[h + p + 1]));
        ms[p] += t;
      }
    return KQ_OK;
  }
  ~PhaseTimer() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

// One half step: F_out = sum_t (|U s2_t|^2 / (T k2)) s1_t s1_t^T, U from M (k2 x k2).
kq_status half_step(const float* M, const uint16_t* S2, int64_t ld2, int64_t k2, const uint16_t* S1,
                    int64_t ld1, int64_t k1, int64_t T, float* out, const Workspace& w,
                    PhaseTimer& pt, hipStream_t s) {
  KQ_TRY(pt.mark(s));
  KQ_TRY(inverse_factor(M, k2, w, s));
  KQ_TRY(pt.mark(s));
  KQ_TRY(quadratic_forms(S2, ld2, T, k2, w, s));
  KQ_TRY(pt.mark(s));
  const int np = 2 * (int)((k2 + QT - 1) / QT);
  const float c = (float)(1.0 / ((double)T * (double)k2));
  ff_scale_kernel<<<dim3((unsigned)T), dim3(256), 0, s>>>(S1, ld1, (int)k1, w.part, np, c, w.Ss, w.ldS);
  KQ_LAUNCHED("ff_scale_kernel");
  KQ_TRY(pt.mark(s));
  KQ_TRY(gram_lower(w.Ss, w.ldS, S1, ld1, T, k1, out, k1, false, false, s));
  KQ_TRY(gram_lower(w.Ss + k1, w.ldS, S1, ld1, T, k1, out, k1, true, true, s));
  return pt.mark(s);
}

}  // namespace

// U = R^-1 (explicit, upper triangular, k x k, ld k) for M + lambda I = R R^T with
// lambda = damp * mean(diag M) (a zero diagonal counts as 1; its channel is flagged in
// dead): the factorization leaves the diagonal blocks U_JJ and the panels
// P[<J, J] = R[<J, J] U_JJ, and U[<J, J] = -U[<J, <J] P[<J, J] column block by column
// block (fp32 MFMA products, the contraction split over enough workgroups).
kq_status explicit_inverse_factor(const float* M, int64_t k, float damp, float* F, float* Tsc,
                                  uint8_t* dead, double* lam, int* flag, float* U, hipStream_t s) {
  KQ_TRY(damp_and_factor(M, F, Tsc, dead, lam, flag, k, damp, 128, s));
  KQ_TRY(fill_f32(U, k * k, 0.0f, s));
  copy_diag_blocks<<<dim3((unsigned)(k / 128)), dim3(256), 0, s>>>(F, U, k);
  KQ_LAUNCHED("copy_diag_blocks");
  for (int64_t J = 1; J < k / 128; ++J) {
    const int64_t c0 = 128 * J;
    GemmArgs g = {};
    g.M = c0; g.N = 128; g.K = c0;
    g.A = U; g.lda = k; g.transA = false;
    g.B = F + c0; g.ldb = k; g.transB = false;
    g.C = U + c0; g.ldc = k;
    // U is zero there: accumulate, with the contraction split over enough workgroups
    g.alpha = -1.0f; g.accumulate = true; g.upper_only = false;
    g.a_upper = true; g.b_upper = false;
    g.split_k = (int)std::max<int64_t>(1, std::min<int64_t>(16, 256 / J)); g.batch = 1;
    KQ_TRY(gemm_f32(g, s));
  }
  return KQ_OK;
}

}  // namespace kq

extern "C" kq_status kq_flipflop_workspace(int64_t T, int64_t n, int64_t m, size_t* bytes) {
  using namespace kq;
  if (!bytes) return fail(KQ_EINVAL, "kq_flipflop_workspace: bytes is NULL");
  if (T < 1 || n < 128 || m < 128 || n % 128 != 0 || m % 128 != 0 || T > (1ll << 31) ||
      n > (1 << 16) || m > (1 << 16))
    return fail(KQ_ESHAPE, "kq_flipflop_workspace: T >= 1, n and m multiples of 128");
  *bytes = (size_t)layout(T, n, m, nullptr, nullptr);
  return KQ_OK;
}

extern "C" kq_status kq_flipflop(const uint16_t* X, int64_t ldx, const uint16_t* G, int64_t ldg,
                                 int64_t T, int64_t n, int64_t m, int iters, float* A, float* B,
                                 void* ws, size_t ws_bytes, double* phase_ms, void* stream) {
  using namespace kq;
  if (!X || !G || !A || !B || !ws) return fail(KQ_EINVAL, "kq_flipflop: NULL argument");
  size_t need = 0;
  KQ_TRY(kq_flipflop_workspace(T, n, m, &need));
  if (ws_bytes < need) return fail(KQ_EWORKSPACE, "kq_flipflop: workspace of %zu bytes needed", need);
  if (iters < 1 || iters > 1000) return fail(KQ_ESHAPE, "kq_flipflop: iters must be 1 .. 1000");
  if (ldx < n || ldg < m || ldx % 8 != 0 || ldg % 8 != 0 || ((uintptr_t)X & 15) || ((uintptr_t)G & 15))
    return fail(KQ_ESHAPE, "kq_flipflop: leading dims >= the widths, multiples of 8; 16-byte aligned streams");
  Workspace w;
  layout(T, n, m, (char*)ws, &w);
  hipStream_t s = as_stream(stream);
  KQ_HIP(hipMemsetAsync(w.flag, 0, sizeof(int), s));
  identity_kernel<<<dim3((unsigned)ceil_div(m * m, 256)), dim3(256), 0, s>>>(B, m);
  KQ_LAUNCHED("identity_kernel");
  PhaseTimer pt;
  pt.on = phase_ms != nullptr;
  for (int it = 0; it < iters; ++it) {
    KQ_TRY(half_step(B, G, ldg, m, X, ldx, n, T, A, w, pt, s));
    KQ_TRY(half_step(A, X, ldx, n, G, ldg, m, T, B, w, pt, s));
  }
  int flag = 0;
  KQ_HIP(hipMemcpyAsync(&flag, w.flag, sizeof(int), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  if (pt.on) KQ_TRY(pt.read(phase_ms));
  if (flag) return fail(KQ_ENOTSPD, "kq_flipflop: a factor has no Cholesky factor");
  return KQ_OK;
}
