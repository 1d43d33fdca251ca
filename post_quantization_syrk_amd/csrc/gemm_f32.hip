// fp32 matrix products on the matrix cores (v_mfma_f32_32x32x2_f32), used by
// the quantizer: GPTQ's blocked error feedback and the proxy-loss products.
//
// C[M x N] (+)= alpha * op(A) op(B), row-major.  128 x 128 tiles, 256 threads
// (4 waves, each a 64 x 64 sub-tile = 2 x 2 MFMA blocks), 32-deep K stages
// through LDS stored k-major so every MFMA operand read is 32 consecutive
// floats.  Optional split-K (fp32 atomics into C, or one partial product per split
// stored to its own slice), upper-triangle-only tile sets, and a reduction epilogue
// sum(alpha * AB .* D) into an fp64 accumulator.  The direct-to-LDS kernel for plain
// row-major products hands each XCD a contiguous run of tiles in groups of four tile
// columns, so the workgroups that share an L2 also share their operand panels.
#include "device_util.h"
#include "kq_internal.h"

#include <stdlib.h>

namespace kq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int MT = 128, NTL = 128, BK = 32, THREADS = 256;
constexpr int LD_UNITS = MT * BK / 4 / THREADS;   // float4 loads per thread per operand and stage
constexpr int LDA_S = MT + 4, LDB_S = NTL + 4;

struct Args {
  int64_t M, N, K;
  const float* A; int64_t lda; int transA;
  const float* B; int64_t ldb; int transB;
  float* C; int64_t ldc;
  float alpha;
  int accumulate, upper_only, a_upper, b_upper, split_k;
  int64_t partial_stride;
  int64_t k_per_split;
  int64_t strideA, strideB, strideC;
  const float* D; int64_t ldd; double* red;
};

// Loads one BK-deep stage of op(A) (MT x BK) into registers: LD_UNITS float4 per thread.
__device__ __forceinline__ void load_a(const Args& a, int64_t m0, int64_t k0, int64_t kend,
                                       float4 (&r)[LD_UNITS]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < LD_UNITS; ++u) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!a.transA) {
      // A row-major M x K: thread -> row (t/8 + 32u), k quad (t%8)
      const int64_t row = m0 + (t >> 3) + 32 * u;
      const int64_t k = k0 + 4 * (t & 7);
      if (row < a.M && k < kend) v = *(const float4*)(a.A + row * a.lda + k);
    } else {
      // A stored K x M: thread -> k (t/32 + 8u), m quad (t%32)
      const int64_t k = k0 + (t >> 5) + 8 * u;
      const int64_t col = m0 + 4 * (t & 31);
      if (k < kend && col < a.M) v = *(const float4*)(a.A + k * a.lda + col);
    }
    r[u] = v;
  }
}

__device__ __forceinline__ void load_b(const Args& a, int64_t n0, int64_t k0, int64_t kend,
                                       float4 (&r)[LD_UNITS]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < LD_UNITS; ++u) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!a.transB) {
      // B row-major K x N: thread -> k (t/32 + 8u), n quad (t%32)
      const int64_t k = k0 + (t >> 5) + 8 * u;
      const int64_t col = n0 + 4 * (t & 31);
      if (k < kend && col < a.N) v = *(const float4*)(a.B + k * a.ldb + col);
    } else {
      // B stored N x K: thread -> n row (t/8 + 32u), k quad (t%8)
      const int64_t row = n0 + (t >> 3) + 32 * u;
      const int64_t k = k0 + 4 * (t & 7);
      if (row < a.N && k < kend) v = *(const float4*)(a.B + row * a.ldb + k);
    }
    r[u] = v;
  }
}

// Stores a stage k-major: As[k][m], Bs[k][n]
__device__ __forceinline__ void store_a(const Args& a, float* As, const float4 (&r)[LD_UNITS]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < LD_UNITS; ++u) {
    if (!a.transA) {
      const int m = (t >> 3) + 32 * u, k = 4 * (t & 7);
      As[(k + 0) * LDA_S + m] = r[u].x;
      As[(k + 1) * LDA_S + m] = r[u].y;
      As[(k + 2) * LDA_S + m] = r[u].z;
      As[(k + 3) * LDA_S + m] = r[u].w;
    } else {
      const int k = (t >> 5) + 8 * u, m = 4 * (t & 31);
      *(float4*)(As + k * LDA_S + m) = r[u];
    }
  }
}

__device__ __forceinline__ void store_b(const Args& a, float* Bs, const float4 (&r)[LD_UNITS]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < LD_UNITS; ++u) {
    if (!a.transB) {
      const int k = (t >> 5) + 8 * u, n = 4 * (t & 31);
      *(float4*)(Bs + k * LDB_S + n) = r[u];
    } else {
      const int n = (t >> 3) + 32 * u, k = 4 * (t & 7);
      Bs[(k + 0) * LDB_S + n] = r[u].x;
      Bs[(k + 1) * LDB_S + n] = r[u].y;
      Bs[(k + 2) * LDB_S + n] = r[u].z;
      Bs[(k + 3) * LDB_S + n] = r[u].w;
    }
  }
}

__global__ __launch_bounds__(THREADS) void gemm_f32_kernel(Args a) {
  const int64_t tm = blockIdx.x, tn = blockIdx.y;
  if (a.upper_only && tm > tn) return;
  const int64_t m0 = tm * MT, n0 = tn * NTL;
  const int bz = blockIdx.z / a.split_k;           // batch index
  const int sz = blockIdx.z % a.split_k;           // split index
  a.A += bz * a.strideA;
  a.B += bz * a.strideB;
  a.C += bz * a.strideC;
  int64_t kbeg = (int64_t)sz * a.k_per_split;
  int64_t kend = min(a.K, kbeg + a.k_per_split);
  // upper-triangular A: rows >= m0 are zero for k < m0
  if (a.a_upper && kbeg < m0) kbeg = min(kend, (m0 / BK) * BK);
  // upper-triangular B: columns < n0 + NTL are zero for k >= n0 + NTL
  if (a.b_upper) kend = max(kbeg, min(kend, n0 + NTL));
  if (kbeg >= kend && a.split_k > 1) return;

  __shared__ __attribute__((aligned(16))) float As[2][BK * LDA_S];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB_S];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int l32 = lane & 31, kh = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nst = (int)((kend - kbeg + BK - 1) / BK);
  float4 ra[LD_UNITS], rb[LD_UNITS];
  if (nst > 0) {
    load_a(a, m0, kbeg, kend, ra);
    load_b(a, n0, kbeg, kend, rb);
    store_a(a, As[0], ra);
    store_b(a, Bs[0], rb);
  }
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nst;
    if (more) {
      load_a(a, m0, kbeg + (int64_t)(s + 1) * BK, kend, ra);
      load_b(a, n0, kbeg + (int64_t)(s + 1) * BK, kend, rb);
    }
    const float* as = As[buf];
    const float* bs = Bs[buf];
    // all operands of the stage are read before the multiplies, so the LDS latency is paid
    // once per stage instead of once per k step
    float av[BK / 2][2], bv[BK / 2][2];
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) av[kk][i] = as[(2 * kk + kh) * LDA_S + wm + 32 * i + l32];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[kk][j] = bs[(2 * kk + kh) * LDB_S + wn + 32 * j + l32];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
    if (more) {
      store_a(a, As[buf ^ 1], ra);
      store_b(a, Bs[buf ^ 1], rb);
    }
    __syncthreads();
  }

  const int rh = kh * 4;
  if (a.red) {
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          if (row < a.M && col < a.N)
            part += (double)(a.alpha * acc[i][j][r]) * (double)a.D[row * a.ldd + col];
        }
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) atomicAdd(a.red, part);
    return;
  }
  if (a.partial_stride > 0) {
    float* Cp = a.C + (int64_t)sz * a.partial_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          if (row < a.M) Cp[row * a.ldc + col] = a.alpha * acc[i][j][r];
        }
      }
    return;
  }
  if (a.split_k > 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          if (row < a.M) atomicAdd(a.C + row * a.ldc + col, a.alpha * acc[i][j][r]);
        }
      }
    return;
  }
  // C += alpha AB: every C value of the thread is loaded before any is stored, so the
  // loads are issued together instead of one round trip per element.
  if (a.accumulate) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          const float c = (row < a.M && col < a.N) ? a.C[row * a.ldc + col] : 0.0f;
          acc[i][j][r] = fmaf(a.alpha, acc[i][j][r], c);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] *= a.alpha;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn + 32 * j + l32;
      if (col >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
        if (row < a.M) a.C[row * a.ldc + col] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Direct-to-LDS kernel for C (+)= alpha A B with A row-major M x K and B row-major K x N (the
// GPTQ feedback product).  Both tiles are copied into LDS as they lie in memory by the load
// unit (global_load_lds, 16 bytes per lane) into a ring of four 32-deep K stages (128 KB).
// The MFMA (v_mfma_f32_32x32x2f32) sums over its two k slots, so the lane half h of every
// k step can take any true k as long as A and B agree: half h takes k = 16 h + s for the
// 16 steps s of a stage.  A lane then needs 16 consecutive floats of one A row (four 16-byte
// reads) and 16 rows of one B column.  A rows (32 floats) hold their 16-byte chunks at slot
// chunk ^ ((row >> 1) & 7), B rows (128 floats) at chunk ^ (8 * ((k >> 4) & 1)), which
// makes both reads conflict-free.  Chunks outside the matrix are read from a zero chunk, so
// every wave issues the same number of copies per stage and the vmcnt waits are exact.
// ---------------------------------------------------------------------------------------------
constexpr int DBK = 32;               // k per stage
constexpr int DSA = MT * DBK;         // floats of the A tile of a stage
constexpr int DSB = DBK * NTL;        // floats of the B tile of a stage
constexpr int DSTG = DSA + DSB;       // 32 KB per stage
constexpr int DRING = 4;

__device__ __attribute__((aligned(16))) float g_zero_chunk_f32[4];

struct DArgs {
  int64_t M, N, K;
  const float* A; int64_t lda;
  const float* B; int64_t ldb;
  float* C; int64_t ldc;
  float alpha;
  int accumulate, split_k;
  int upper_only;     // only tiles with tile row <= tile column
  int64_t k_per_split;
  int64_t partial_stride;
  int tm, tn, gn;      // tile rows, tile columns, tile columns per group
  int xcds;
  int64_t per_split, total, per_xcd;
};

// Tile o of one split's list.  Tiles come in groups of gn tile columns; inside a group, tile
// rows in order with the group's columns adjacent, so the workgroups an XCD runs at once cover
// a compact block of C and share their A and B panels in its L2.  Upper sets (tile row <= tile
// column, tm >= tn) keep in each group the rows up to the group's last column.
__device__ __forceinline__ void dma_tile(const DArgs& a, int64_t o, int& ti, int& tj) {
  if (!a.upper_only) {
    const int64_t gsz = (int64_t)a.gn * a.tm;
    const int g = (int)(o / gsz);
    const int c0 = g * a.gn, w = min(a.gn, a.tn - c0);
    const int r = (int)(o - g * gsz);
    ti = r / w;
    tj = c0 + r % w;
    return;
  }
  int64_t base = 0;
  for (int g = 0;; ++g) {
    const int c0 = g * a.gn, w = min(a.gn, a.tn - c0);
    const int64_t full = (int64_t)w * (c0 + 1);
    const int64_t cnt = full + w * (w - 1) / 2;
    if (o < base + cnt) {
      int r = (int)(o - base);
      if (r < full) {
        ti = r / w;
        tj = c0 + r % w;
      } else {
        r -= (int)full;
        int k = 1;
        while (r >= w - k) { r -= w - k; ++k; }
        ti = c0 + k;
        tj = c0 + k + r;
      }
      return;
    }
    base += cnt;
  }
}

__device__ __forceinline__ void gcopy(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst,
                                   16, 0, 0);
}

__global__ __launch_bounds__(THREADS) void gemm_nn_dma_kernel(DArgs a) {
  __shared__ __attribute__((aligned(1024))) float r0[DSTG];
  __shared__ __attribute__((aligned(1024))) float r1[DSTG];
  __shared__ __attribute__((aligned(1024))) float r2[DSTG];
  __shared__ __attribute__((aligned(1024))) float r3[DSTG];
  // workgroup u runs on XCD u mod xcds, which takes the items xcd * per_xcd .. + per_xcd - 1
  const int64_t u = blockIdx.x;
  const int64_t item = (u % a.xcds) * a.per_xcd + u / a.xcds;
  if (item >= a.total) return;
  const int split = (int)(item / a.per_split);
  int ti, tj;
  dma_tile(a, item - split * a.per_split, ti, tj);
  const int64_t m0 = (int64_t)ti * MT, n0 = (int64_t)tj * NTL;
  const int64_t kbeg = (int64_t)split * a.k_per_split;
  const int64_t kend = min(a.K, kbeg + a.k_per_split);
  if (kbeg >= kend) return;
  const int nst = (int)((kend - kbeg + DBK - 1) / DBK);   // stages of this split
  const int nfull = nst / DRING * DRING;                   // in whole turns of the ring
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const float* zero = g_zero_chunk_f32;

  // copy sources (stage-invariant parts): A instruction r of wave w covers rows 8p..8p+7,
  // p = 4w + r; B instruction r covers k rows 2p, 2p+1
  uint32_t offA[4], offB[4];
  int chA[4], krB[4];
  bool okA[4], okB[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = 4 * wave + r;
    const int m = 8 * p + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    chA[r] = c;
    offA[r] = (uint32_t)(m * a.lda + 4 * c);
    okA[r] = m0 + m < a.M;
    const int kr = 2 * p + (lane >> 5);
    const int cb = (lane & 31) ^ (((kr >> 4) & 1) << 3);
    krB[r] = kr;
    offB[r] = (uint32_t)(kr * a.ldb + 4 * cb);
    okB[r] = n0 + 4 * cb < a.N;
  }
  const float* Abase = a.A + m0 * a.lda;
  const float* Bbase = a.B + n0;
  auto issue = [&](int st, float* buf) {
    const int64_t k0 = kbeg + (int64_t)st * DBK;
    const float* ab = Abase + min(k0, kend);
    const float* bb = Bbase + min(k0, kend) * a.ldb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool v = okA[r] && k0 + 4 * chA[r] < kend;
      gcopy(v ? ab + offA[r] : zero, buf + (4 * wave + r) * 256);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool v = okB[r] && k0 + krB[r] < kend;
      gcopy(v ? bb + offB[r] : zero, buf + DSA + (4 * wave + r) * 256);
    }
  };

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  // operand read offsets (floats) inside a stage buffer
  int oa[2][4], ob[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = wm + 32 * i + l32;
#pragma unroll
    for (int t = 0; t < 4; ++t) oa[i][t] = m * DBK + 4 * ((4 * h + t) ^ ((m >> 1) & 7));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = wn + 32 * j + l32;
    ob[j] = DSA + 16 * h * NTL + 4 * ((n >> 2) ^ (h << 3)) + (n & 3);
  }
  float xa[2][16], xb[2][16], ya[2][16], yb[2][16];
  auto read = [&](const float* buf, float (&av)[2][16], float (&bv)[2][16]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 v = *(const float4*)(buf + oa[i][t]);
        av[i][4 * t] = v.x; av[i][4 * t + 1] = v.y; av[i][4 * t + 2] = v.z; av[i][4 * t + 3] = v.w;
      }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) bv[j][s2] = buf[ob[j] + s2 * NTL];
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto mma = [&](const float (&av)[2][16], const float (&bv)[2][16]) {
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s2], bv[j][s2], acc[i][j], 0, 0, 0);
  };

  issue(0, r0);
  issue(1, r1);
  issue(2, r2);
  issue(3, r3);
  __builtin_amdgcn_s_waitcnt(wait_vm(16));   // stages 0 and 1 of this wave
  lds_barrier();
  read(r0, xa, xb);
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  lds_barrier();

  // Step s (operands of stage s in registers, stage s+1 visible): refill stage s's buffer
  // with stage s + 4, multiply stage s while reading stage s+1, wait for this wave's copies of
  // stage s+2 and every wave's reads of stage s+1.
#define KQ_G_STEP(J, CUR, NXT, RA, RB, NA, NB)                     \
  {                                                                \
    issue(s0 + (J) + DRING, CUR);                                  \
    read(NXT, NA, NB);                                             \
    mma(RA, RB);                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {             \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
    }                                                              \
    __builtin_amdgcn_sched_barrier(0);                             \
    __builtin_amdgcn_s_waitcnt(wait_vm(16));                      \
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);                       \
    lds_barrier();                                                    \
  }
  for (int s0 = 0; s0 < nfull; s0 += DRING) {
    KQ_G_STEP(0, r0, r1, xa, xb, ya, yb)
    KQ_G_STEP(1, r1, r2, ya, yb, xa, xb)
    KQ_G_STEP(2, r2, r3, xa, xb, ya, yb)
    KQ_G_STEP(3, r3, r0, ya, yb, xa, xb)
  }
  {
    // the last nst % DRING stages (uniform branches; copies past kend read the zero chunk)
    const int s0 = nfull;
    if (nst > s0) KQ_G_STEP(0, r0, r1, xa, xb, ya, yb)
    if (nst > s0 + 1) KQ_G_STEP(1, r1, r2, ya, yb, xa, xb)
    if (nst > s0 + 2) KQ_G_STEP(2, r2, r3, xa, xb, ya, yb)
  }
#undef KQ_G_STEP
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  const int kh = h, rh = kh * 4;
  if (a.partial_stride > 0) {
    float* Cp = a.C + (int64_t)split * a.partial_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          if (row < a.M) Cp[row * a.ldc + col] = a.alpha * acc[i][j][r];
        }
      }
    return;
  }
  if (a.split_k > 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          if (row < a.M) atomicAdd(a.C + row * a.ldc + col, a.alpha * acc[i][j][r]);
        }
      }
    return;
  }
  if (a.accumulate) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn + 32 * j + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
          const float c = (row < a.M && col < a.N) ? a.C[row * a.ldc + col] : 0.0f;
          acc[i][j][r] = fmaf(a.alpha, acc[i][j][r], c);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] *= a.alpha;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn + 32 * j + l32;
      if (col >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + rh + (r & 3);
        if (row < a.M) a.C[row * a.ldc + col] = acc[i][j][r];
      }
    }
}

}  // namespace

kq_status gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return KQ_OK;
  const bool partial = g.partial_stride > 0;
  if (g.split_k < 1 || (g.split_k > 1 && !g.accumulate && !g.red && !partial))
    return fail(KQ_EINVAL, "gemm_f32: split_k > 1 needs accumulation or partial slices");
  if (partial && (g.accumulate || g.red || g.batch > 1 || g.upper_only || g.a_upper || g.b_upper ||
                  g.K <= 0 || g.partial_stride < g.M * g.ldc))
    return fail(KQ_EINVAL, "gemm_f32: partial slices need a plain product with K > 0");
  // plain row-major products with 16-byte aligned rows take the direct-to-LDS kernel
  const bool aligned = ((uintptr_t)g.A % 16 == 0) && ((uintptr_t)g.B % 16 == 0) &&
                       g.lda % 4 == 0 && g.ldb % 4 == 0 && g.K % 4 == 0 && g.N % 4 == 0;
  // (upper tile sets there need at least as many tile rows as tile columns)
  if (!g.transA && !g.transB && !g.a_upper && !g.b_upper && !g.red &&
      (g.batch <= 1) && aligned && g.K > 0 && 128 * g.lda + (int64_t)DBK * g.ldb < ((int64_t)1 << 32) &&
      (!g.upper_only || g.M >= g.N)) {
    DArgs d;
    d.M = g.M; d.N = g.N; d.K = g.K;
    d.A = g.A; d.lda = g.lda; d.B = g.B; d.ldb = g.ldb; d.C = g.C; d.ldc = g.ldc;
    d.alpha = g.alpha; d.accumulate = g.accumulate; d.upper_only = g.upper_only ? 1 : 0;
    d.k_per_split = ceil_div(ceil_div(g.K, g.split_k), DBK) * DBK;
    d.split_k = (int)ceil_div(g.K, d.k_per_split);
    d.partial_stride = g.partial_stride;
    if (g.splits_used) *g.splits_used = d.split_k;
    d.tm = (int)ceil_div(g.M, MT);
    d.tn = (int)ceil_div(g.N, NTL);
    d.gn = 4;
    d.per_split = g.upper_only ? (int64_t)d.tn * (d.tn + 1) / 2 : (int64_t)d.tm * d.tn;
    d.total = d.per_split * d.split_k;
    d.xcds = device_cu_count() % 8 == 0 ? 8 : 1;
    d.per_xcd = ceil_div(d.total, d.xcds);
    if (d.per_xcd * d.xcds > 0x7fffffff) return fail(KQ_ESHAPE, "gemm_f32: too many tiles");
    gemm_nn_dma_kernel<<<dim3((unsigned)(d.per_xcd * d.xcds)), dim3(THREADS), 0, s>>>(d);
    KQ_LAUNCHED("gemm_nn_dma_kernel");
    return KQ_OK;
  }
  Args a;
  a.M = g.M; a.N = g.N; a.K = g.K;
  a.A = g.A; a.lda = g.lda; a.transA = g.transA;
  a.B = g.B; a.ldb = g.ldb; a.transB = g.transB;
  a.C = g.C; a.ldc = g.ldc; a.alpha = g.alpha;
  a.accumulate = g.accumulate; a.upper_only = g.upper_only; a.a_upper = g.a_upper;
  a.b_upper = g.b_upper; a.split_k = g.split_k;
  a.strideA = g.strideA; a.strideB = g.strideB; a.strideC = g.strideC;
  const int batch = g.batch > 0 ? g.batch : 1;
  if (batch > 1 && g.red) return fail(KQ_EINVAL, "gemm_f32: batched reduction not supported");
  a.D = g.D; a.ldd = g.ldd; a.red = g.red;
  a.k_per_split = ceil_div(ceil_div(g.K > 0 ? g.K : 1, g.split_k), BK) * BK;
  const int splits = g.K > 0 ? (int)ceil_div(g.K, a.k_per_split) : 1;
  // one split left: a plain read-add-write gives the same C += alpha AB
  a.split_k = splits;
  a.partial_stride = g.partial_stride;
  if (g.splits_used) *g.splits_used = splits;
  dim3 grid((unsigned)ceil_div(g.M, MT), (unsigned)ceil_div(g.N, NTL), (unsigned)(splits * batch));
  gemm_f32_kernel<<<grid, dim3(THREADS), 0, s>>>(a);
  KQ_LAUNCHED("gemm_f32_kernel");
  return KQ_OK;
}

}  // namespace kq
