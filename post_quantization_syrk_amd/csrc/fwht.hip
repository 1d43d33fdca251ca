// Bidirectional incoherence processing (BiIP): rescale + randomized Hadamard
// rotation of W, H_X and H_G on the input and the output side.
//
// KronQ README, opening section: the incoherence rotation and the rescale act on the
// input side and on the output side; flags table: --incoh_kernel had, --alpha 0.25;
// KronQ arXiv abstract, point 1: the input-side random rotation is extended
// to the output dimension using the gradient covariance.
//
// With P = blockdiag(Had_b) diag(S) / sqrt(b) (Sylvester Hadamard, natural
// order) and rescale vectors d_in, d_out:
//   W~   = P_out D_out W D_in P_in^T
//   H~_X = P_in D_in^-1 H_X D_in^-1 P_in^T,   H~_G = P_out D_out^-1 H_G D_out^-1 P_out^T
// All diagonal factors (rescale, signs, 1/sqrt(b)) are folded into the loads
// of one row pass; the transform along the strided (row) index is done by
// tiled column passes.  Every pass reads and writes each element once.
//
// Row pass, 4096-element blocks: three rounds of 4 index bits in registers with two LDS
// regroupings (row_fwht4096_kernel); 8192-element blocks likewise with rounds of 5, 5 and 3
// bits (row_fwht8192_kernel).
// Row pass, other blocks (wavefront-shuffle FWHT): a Hadamard block of b contiguous
// elements is spread over b/EPT threads with EPT values each (16-byte
// vectors).  Butterflies over the in-register index bits run in registers,
// over the lane bits with cross-lane xor shuffles, and over the wave bits
// (blocks longer than 64 * EPT) through LDS.
// Column pass: a tile of R = 2^mb rows (stride 2^k0) x 64 columns; each
// thread holds 4 columns x R/16 rows, butterflies the register bits, then
// one LDS transpose brings the remaining row bits into registers.
#include "device_util.h"
#include "kq_internal.h"

#include <math.h>

namespace kq {
namespace {

constexpr int NT = 256;

// ---------------------------------------------------------------------------
// norms and rescale vectors
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Both squared-norm vectors of W from one read of it.  A workgroup takes NR_ROWS whole rows;
// thread t reads the 16-byte column chunks 4t + 1024 j of each row.
//   rowsum[r] = sum_i W[r][i]^2: per-thread partial sums, then a fixed reduction order
//               (wave shuffles, then the four waves' values), stored directly (deterministic);
//   colsum[i] += sum over the workgroup's rows of W[r][i]^2 (atomics; colsum pre-zeroed).
// Either output may be NULL.  Rows past `out` and chunks past `in` read 0 (buffer offsets out
// of range), so no load sits behind a branch.
constexpr int NR_ROWS = 32;
template <int J>
__global__ __launch_bounds__(NT) void norms_kernel(const float* __restrict__ W, int64_t out,
                                                   int64_t in, float* __restrict__ colsum,
                                                   float* __restrict__ rowsum) {
  // rows in flight per unrolled step: about 16 chunk loads per thread
  constexpr int UR = J <= 2 ? 8 : J <= 4 ? 4 : J <= 8 ? 2 : 1;
  __shared__ float part[NT / 64][NR_ROWS];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * NR_ROWS;
  const __amdgpu_buffer_rsrc_t rr = rsrc(W + r0 * in);
  float4 cacc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) cacc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll UR
  for (int k = 0; k < NR_ROWS; ++k) {
    u32x4 q[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t c = 4 * t + 1024 * j;
      const bool ok = r0 + k < out && c < in;
      q[j] = __builtin_amdgcn_raw_buffer_load_b128(rr, ok ? (int)(((int64_t)k * in + c) * 4) : OOB, 0, 0);
    }
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float a = __uint_as_float(q[j].x), b = __uint_as_float(q[j].y);
      const float c = __uint_as_float(q[j].z), d = __uint_as_float(q[j].w);
      cacc[j].x += a * a; cacc[j].y += b * b; cacc[j].z += c * c; cacc[j].w += d * d;
      rs += a * a + b * b + c * c + d * d;
    }
    rs = wave_sum(rs);
    if ((t & 63) == 0) part[t >> 6][k] = rs;
  }
  if (colsum) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t c = 4 * t + 1024 * j;
      if (c < in) {
        atomicAdd(colsum + c + 0, cacc[j].x);
        atomicAdd(colsum + c + 1, cacc[j].y);
        atomicAdd(colsum + c + 2, cacc[j].z);
        atomicAdd(colsum + c + 3, cacc[j].w);
      }
    }
  }
  if (rowsum) {
    __syncthreads();
    if (t < NR_ROWS && r0 + t < out)
      rowsum[r0 + t] = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
  }
}

kq_status launch_norms(const float* W, int64_t out, int64_t in, float* colsum, float* rowsum,
                       hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(out, NR_ROWS));
  switch (ceil_div(in, 1024)) {
#define KQ_NORMS_CASE(X) \
  case X: norms_kernel<X><<<grid, dim3(NT), 0, s>>>(W, out, in, colsum, rowsum); break;
    KQ_NORMS_CASE(1) KQ_NORMS_CASE(2) KQ_NORMS_CASE(3) KQ_NORMS_CASE(4) KQ_NORMS_CASE(5)
    KQ_NORMS_CASE(6) KQ_NORMS_CASE(7) KQ_NORMS_CASE(8) KQ_NORMS_CASE(9) KQ_NORMS_CASE(10)
    KQ_NORMS_CASE(11) KQ_NORMS_CASE(12) KQ_NORMS_CASE(13) KQ_NORMS_CASE(14) KQ_NORMS_CASE(15)
    KQ_NORMS_CASE(16)
#undef KQ_NORMS_CASE
    default: return KQ_ENOTIMPL;
  }
  KQ_LAUNCHED("norms_kernel");
  return KQ_OK;
}

// Two-pass fallback for rows longer than 16384: colsum over stripes of 32 rows (atomics),
// rowsum one workgroup per row.
__global__ __launch_bounds__(NT) void col_sumsq_kernel(const float* __restrict__ W, int64_t out,
                                                       int64_t in, float* __restrict__ colsum) {
  const int64_t c = ((int64_t)blockIdx.x * NT + threadIdx.x) * 4;
  if (c >= in) return;
  const int64_t r0 = (int64_t)blockIdx.y * NR_ROWS;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < NR_ROWS && r0 + k < out; ++k) {
    const float4 v = *(const float4*)(W + (r0 + k) * in + c);
    acc.x += v.x * v.x; acc.y += v.y * v.y; acc.z += v.z * v.z; acc.w += v.w * v.w;
  }
  atomicAdd(colsum + c + 0, acc.x);
  atomicAdd(colsum + c + 1, acc.y);
  atomicAdd(colsum + c + 2, acc.z);
  atomicAdd(colsum + c + 3, acc.w);
}

__global__ __launch_bounds__(NT) void row_sumsq_kernel(const float* __restrict__ W, int64_t in,
                                                       float* __restrict__ rowsum) {
  const float* row = W + (int64_t)blockIdx.x * in;
  float acc = 0.f;
  for (int64_t c = threadIdx.x * 4; c < in; c += NT * 4) {
    float4 v = *(const float4*)(row + c);
    acc += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  acc = wave_sum(acc);
  __shared__ float part[NT / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) rowsum[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

// colsum (pre-zeroed) and / or rowsum of W, from one read of W where the row fits the fused
// kernel.
kq_status squared_norms(const float* W, int64_t out, int64_t in, float* colsum, float* rowsum,
                        hipStream_t s) {
  if (in <= 16 * 1024 && (int64_t)NR_ROWS * in * 4 < ((int64_t)1 << 31))
    return launch_norms(W, out, in, colsum, rowsum, s);
  if (colsum) {
    dim3 grid((unsigned)ceil_div(in / 4, NT), (unsigned)ceil_div(out, NR_ROWS));
    col_sumsq_kernel<<<grid, dim3(NT), 0, s>>>(W, out, in, colsum);
    KQ_LAUNCHED("col_sumsq_kernel");
  }
  if (rowsum) {
    row_sumsq_kernel<<<dim3((unsigned)out), dim3(NT), 0, s>>>(W, in, rowsum);
    KQ_LAUNCHED("row_sumsq_kernel");
  }
  return KQ_OK;
}

// d[i] = (H[i,i] / norm[i])^alpha, 1 where either is not positive (in place over norm)
__global__ void rescale_kernel(const float* __restrict__ H, int64_t n, float* __restrict__ d,
                               float alpha) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double h = (double)H[i * n + i];
  const double c = (double)d[i];
  d[i] = (h > 0.0 && c > 0.0) ? (float)pow(h / c, (double)alpha) : 1.0f;
}

// ---------------------------------------------------------------------------
// row pass
// ---------------------------------------------------------------------------
struct Scale {
  const float* d;       // rescale vector or NULL
  const int8_t* sign;   // +-1 or NULL
  int invert;           // use 1/d instead of d
  float mul;            // constant factor (1/sqrt(b))
};

// Branch-free (a branch here would let the compiler sink loads issued before it past it):
// mul * d, mul / d or mul from the raw d word, negated when the sign bit is set.
__device__ __forceinline__ float factor_of(const Scale& s, unsigned dword, bool neg) {
  const bool hd = s.d != nullptr, hs = s.sign != nullptr;
  const bool mul_d = hd && !s.invert, div_d = hd && s.invert;
  const float d = __uint_as_float(dword);
  const float v = (s.mul * (mul_d ? d : 1.f)) / (div_d ? d : 1.f);
  return hs && neg ? -v : v;
}

// The factors of the 16 consecutive entries i0 + c .. i0 + c + 15 (c a multiple of 16): four
// 16-byte loads of d and one of the signs (a missing vector is read out of range, as 0).
struct ScaleLoads16 {
  u32x4 d[4];
  u32x4 g;
};

__device__ __forceinline__ void scales16_issue(const Scale& s, int64_t i0, int c,
                                               ScaleLoads16& L) {
  const bool hd = s.d != nullptr, hs = s.sign != nullptr;
  const __amdgpu_buffer_rsrc_t rd = rsrc(hd ? s.d + i0 : s.d), rg = rsrc(hs ? s.sign + i0 : s.sign);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    L.d[q] = __builtin_amdgcn_raw_buffer_load_b128(rd, hd ? 4 * (c + 4 * q) : OOB, 0, 0);
  L.g = __builtin_amdgcn_raw_buffer_load_b128(rg, hs ? c : OOB, 0, 0);
}

__device__ __forceinline__ void scales16_form(const Scale& s, const ScaleLoads16& L,
                                              float (&out)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k)
    out[k] = factor_of(s, L.d[k >> 2][k & 3], ((L.g[k >> 2] >> (8 * (k & 3) + 7)) & 1u) != 0);
}

// The factors of R consecutive rows r0 .. r0 + R - 1 (rows at or past `rows` get any value):
// one word of d and the word holding the sign byte per row.  The sign words are read at
// 4-byte-aligned offsets within the vector, whose length is a multiple of 4, so no read
// passes its end.  Raw words: their use comes after the other loads have been issued.
template <int R>
struct RowLoads {
  unsigned d[R];
  unsigned g[R];
};

template <int R>
__device__ __forceinline__ void rows_issue(const Scale& s, int64_t r0, int64_t rows,
                                          RowLoads<R>& L) {
  const bool hd = s.d != nullptr, hs = s.sign != nullptr;
  const __amdgpu_buffer_rsrc_t rd = rsrc(hd ? s.d + r0 : s.d);
  const __amdgpu_buffer_rsrc_t rg = rsrc(hs ? s.sign + (r0 & ~(int64_t)3) : s.sign);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool ok = r0 + k < rows;
    const int rel = (int)(r0 & 3) + k;
    L.d[k] = __builtin_amdgcn_raw_buffer_load_b32(rd, hd && ok ? 4 * k : OOB, 0, 0);
    L.g[k] = __builtin_amdgcn_raw_buffer_load_b32(rg, hs && ok ? (rel & ~3) : OOB, 0, 0);
  }
}

template <int R>
__device__ __forceinline__ void rows_form(const Scale& s, int64_t r0, const RowLoads<R>& L,
                                          float (&out)[R]) {
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int rel = (int)(r0 & 3) + k;
    out[k] = factor_of(s, L.d[k], ((L.g[k] >> (8 * (rel & 3) + 7)) & 1u) != 0);
  }
}

__device__ __forceinline__ float scale_at(const Scale& s, int64_t i) {
  float v = s.mul;
  if (s.d) v = s.invert ? v / s.d[i] : v * s.d[i];
  if (s.sign) v = s.sign[i] < 0 ? -v : v;
  return v;
}

template <int EPT>
__global__ __launch_bounds__(NT) void row_fwht_kernel(const float* __restrict__ src,
                                                      float* __restrict__ dst, int64_t rows,
                                                      int64_t n, int b, Scale rs, Scale cs) {
  extern __shared__ float sm[];
  const int TPR = b / EPT;               // threads per Hadamard block (power of 2, <= 256)
  const int BPW = NT / TPR;              // blocks per workgroup
  const int tid = threadIdx.x;
  const int lb = tid / TPR, tb = tid % TPR;
  const int64_t blocks_per_row = n / b;
  const int64_t g = (int64_t)blockIdx.x * BPW + lb;
  const bool active = g < rows * blocks_per_row;
  const int64_t r = active ? g / blocks_per_row : 0;
  const int64_t c0 = active ? (g % blocks_per_row) * b : 0;

  // Every load is issued before any value is used, with no branch around them (a branch
  // would make each wait for the ones before it): a thread of an inactive block reads block 0
  // of row 0 and stores nothing; a missing scale vector reads as 0 through an out-of-range
  // offset, which factor_of ignores.
  float v[EPT];
  {
    const bool rhd = rs.d != nullptr, rhs = rs.sign != nullptr;
    const bool chd = cs.d != nullptr, chs = cs.sign != nullptr;
    const __amdgpu_buffer_rsrc_t rrd = rsrc(rs.d), rrg = rsrc(rs.sign);
    const __amdgpu_buffer_rsrc_t rcd = rsrc(cs.d), rcg = rsrc(cs.sign);
    const unsigned rdw = __builtin_amdgcn_raw_buffer_load_b32(rrd, rhd ? (int)(4 * r) : OOB, 0, 0);
    const unsigned rgb = __builtin_amdgcn_raw_buffer_load_b8(rrg, rhs ? (int)r : OOB, 0, 0);
    const float* p = src + r * n + c0;
    float4 qv[EPT / 4];
    u32x4 cd[EPT / 4];
    unsigned cg[EPT / 4];
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      const int x = 4 * tb + 4 * TPR * j;
      qv[j] = *(const float4*)(p + x);
      cd[j] = __builtin_amdgcn_raw_buffer_load_b128(rcd, chd ? (int)(4 * (c0 + x)) : OOB, 0, 0);
      cg[j] = __builtin_amdgcn_raw_buffer_load_b32(rcg, chs ? (int)(c0 + x) : OOB, 0, 0);
    }
    const float rsc = factor_of(rs, rdw, (rgb & 0x80u) != 0);
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      v[4 * j + 0] = qv[j].x * rsc * factor_of(cs, cd[j][0], ((cg[j] >> 7) & 1u) != 0);
      v[4 * j + 1] = qv[j].y * rsc * factor_of(cs, cd[j][1], ((cg[j] >> 15) & 1u) != 0);
      v[4 * j + 2] = qv[j].z * rsc * factor_of(cs, cd[j][2], ((cg[j] >> 23) & 1u) != 0);
      v[4 * j + 3] = qv[j].w * rsc * factor_of(cs, cd[j][3], ((cg[j] >> 31) & 1u) != 0);
    }
  }
  // register bits: e = 4j + q  <->  x = q + 4*tb + 4*TPR*j
#pragma unroll
  for (int m = 1; m < EPT; m <<= 1) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (e & m) continue;
      const float a = v[e], c = v[e | m];
      v[e] = a + c;
      v[e | m] = a - c;
    }
  }
  // lane bits of tb (thread index inside the block, within one wave)
  for (int k = 1; k < TPR && k < 64; k <<= 1) {
    const bool hi = (tb & k) != 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float p = __shfl_xor(v[e], k);
      v[e] = hi ? p - v[e] : v[e] + p;
    }
  }
  if (TPR <= 64) {
    if (!active) return;
    float* q = dst + r * n + c0;
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      const int x = 4 * tb + 4 * TPR * j;
      *(float4*)(q + x) = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    }
    return;
  }
  // wave bits: butterflies in LDS over index bits of x at positions 8 .. log2(4*TPR)-1
  float* blk = sm + lb * b;
#pragma unroll
  for (int j = 0; j < EPT / 4; ++j) {
    const int x = 4 * tb + 4 * TPR * j;
    *(float4*)(blk + x) = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  }
  for (int kb = 8; (1 << kb) < 4 * TPR; ++kb) {
    __syncthreads();
    // b/2 pairs per block = b/8 float4 pairs, spread over the TPR threads of the block
    for (int p4 = tb; p4 < b / 8; p4 += TPR) {
      const int pl = p4 * 4;  // pair index of the first of 4 consecutive pairs
      const int lo = ((pl >> kb) << (kb + 1)) | (pl & ((1 << kb) - 1));
      const int hi = lo | (1 << kb);
      float4 a = *(float4*)(blk + lo), c = *(float4*)(blk + hi);
      *(float4*)(blk + lo) = make_float4(a.x + c.x, a.y + c.y, a.z + c.z, a.w + c.w);
      *(float4*)(blk + hi) = make_float4(a.x - c.x, a.y - c.y, a.z - c.z, a.w - c.w);
    }
  }
  __syncthreads();
  if (!active) return;
  float* q = dst + r * n + c0;
#pragma unroll
  for (int j = 0; j < EPT / 4; ++j) {
    const int x = 4 * tb + 4 * TPR * j;
    *(float4*)(q + x) = *(const float4*)(blk + x);
  }
}

// Row pass for 4096-element blocks: one workgroup per (column block, R rows), 16 values per
// thread.  The 12 butterfly stages commute, so they run as three rounds of 4 index bits in
// registers, with the values regrouped through LDS between rounds:
//   round A: x = 16 t + i     (bits 0-3 in registers; contiguous 64-byte loads)
//   round B: x = (t & 15) + 16 i + 256 (t >> 4)
//   round C: x = t + 256 i    (bits 8-11; a wave stores 64 consecutive values per i)
// LDS index x + (x >> 4) keeps the round A writes and round B accesses free of bank conflicts.
// The loads of all R rows are issued at the start (after the scale loads, which are shared
// by every workgroup and come from the cache): a row's transform is short next to the memory
// latency under full load, so a workgroup that fetched one row ahead would wait on every row.
// The thread's 16 column scales are formed once and reused for the workgroup's R rows.
constexpr int RB = 4096;
template <int R>
__global__ __launch_bounds__(NT) void row_fwht4096_kernel(const float* __restrict__ src,
                                                          float* __restrict__ dst, int64_t rows,
                                                          int64_t n, Scale rs, Scale cs) {
  __shared__ float sm[RB + RB / 16];
  const int t = threadIdx.x;
  const int64_t nb = n / RB;
  const int64_t cb = blockIdx.x % nb, r0 = (int64_t)(blockIdx.x / nb) * R;
  const int64_t c0 = cb * RB;
  float csc[16], rsv[R];
  ScaleLoads16 lc;
  RowLoads<R> lr;
  scales16_issue(cs, c0, 16 * t, lc);
  rows_issue<R>(rs, r0, rows, lr);
  // every row's loads (rows past the end read 0), then the factors
  u32x4 in[R][4];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t r = r0 + k;
    const __amdgpu_buffer_rsrc_t rr = rsrc(src + (r < rows ? r : 0) * n + c0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      in[k][j] = __builtin_amdgcn_raw_buffer_load_b128(rr, r < rows ? (16 * t + 4 * j) * 4 : OOB, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  scales16_form(cs, lc, csc);
  rows_form<R>(rs, r0, lr, rsv);
  float v[16];
  auto bfly = [&]() {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e & m) continue;
        const float a = v[e], c = v[e | m];
        v[e] = a + c;
        v[e | m] = a - c;
      }
  };
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t r = r0 + k;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[4 * j] = __uint_as_float(in[k][j].x); v[4 * j + 1] = __uint_as_float(in[k][j].y);
      v[4 * j + 2] = __uint_as_float(in[k][j].z); v[4 * j + 3] = __uint_as_float(in[k][j].w);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= rsv[k] * csc[i];
    bfly();
    if (k > 0) __syncthreads();   // the previous row's round C reads of sm are done
#pragma unroll
    for (int i = 0; i < 16; ++i) sm[17 * t + i] = v[i];   // x = 16 t + i
    __syncthreads();
    const int xb = (t & 15) + 256 * (t >> 4);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int x = xb + 16 * i;
      v[i] = sm[x + (x >> 4)];
    }
    bfly();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int x = xb + 16 * i;
      sm[x + (x >> 4)] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int x = t + 256 * i;
      v[i] = sm[x + (x >> 4)];
    }
    bfly();
    const __amdgpu_buffer_rsrc_t rd = rsrc(dst + (r < rows ? r : 0) * n + c0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[i]), rd,
                                            r < rows ? (t + 256 * i) * 4 : OOB, 0, 0);
  }
}

// Row pass for 8192-element blocks, the same scheme with 32 values per thread: the 13 stages
// as rounds of 5, 5 and 3 index bits in registers with two LDS regroupings,
//   round A: x = 32 t + i                              (bits 0-4; contiguous 128-byte loads)
//   round B: x = (t & 31) + 32 i + 1024 (t >> 5)       (bits 5-9)
//   round C: x = t + 256 i, stages of i's bits 2-4 only (bits 10-12; bits 8-9 are done)
// LDS index x + (x >> 5): the lanes of round A's writes and round B's accesses sit on
// distinct banks (round C's reads put two lanes of a wave on one bank).
constexpr int RB8 = 8192;
template <int R>
__global__ __launch_bounds__(NT) void row_fwht8192_kernel(const float* __restrict__ src,
                                                          float* __restrict__ dst, int64_t rows,
                                                          int64_t n, Scale rs, Scale cs) {
  __shared__ float sm[RB8 + RB8 / 32];
  const int t = threadIdx.x;
  const int64_t nb = n / RB8;
  const int64_t cb = blockIdx.x % nb, r0 = (int64_t)(blockIdx.x / nb) * R;
  const int64_t c0 = cb * RB8;
  float csc[32], rsv[R];
  ScaleLoads16 lc0, lc1;
  RowLoads<R> lr;
  scales16_issue(cs, c0, 32 * t, lc0);
  scales16_issue(cs, c0, 32 * t + 16, lc1);
  rows_issue<R>(rs, r0, rows, lr);
  // every row's loads (rows past the end read 0), then the factors
  u32x4 in[R][8];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t r = r0 + k;
    const __amdgpu_buffer_rsrc_t rr = rsrc(src + (r < rows ? r : 0) * n + c0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      in[k][j] = __builtin_amdgcn_raw_buffer_load_b128(rr, r < rows ? (32 * t + 4 * j) * 4 : OOB, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    float c16[16];
    scales16_form(cs, lc0, c16);
#pragma unroll
    for (int i = 0; i < 16; ++i) csc[i] = c16[i];
    scales16_form(cs, lc1, c16);
#pragma unroll
    for (int i = 0; i < 16; ++i) csc[16 + i] = c16[i];
  }
  rows_form<R>(rs, r0, lr, rsv);
  float v[32];
  // butterfly stages over the register index bits in [m0, 32)
  auto bfly = [&](int m0) {
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      if (m < m0) continue;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if (e & m) continue;
        const float a = v[e], c = v[e | m];
        v[e] = a + c;
        v[e | m] = a - c;
      }
    }
  };
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t r = r0 + k;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[4 * j] = __uint_as_float(in[k][j].x); v[4 * j + 1] = __uint_as_float(in[k][j].y);
      v[4 * j + 2] = __uint_as_float(in[k][j].z); v[4 * j + 3] = __uint_as_float(in[k][j].w);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= rsv[k] * csc[i];
    bfly(1);
    if (k > 0) __syncthreads();   // the previous row's round C reads of sm are done
#pragma unroll
    for (int i = 0; i < 32; ++i) sm[33 * t + i] = v[i];   // x = 32 t + i
    __syncthreads();
    const int xb = (t & 31) + 1024 * (t >> 5);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int x = xb + 32 * i;
      v[i] = sm[x + (x >> 5)];
    }
    bfly(1);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int x = xb + 32 * i;
      sm[x + (x >> 5)] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int x = t + 256 * i;
      v[i] = sm[x + (x >> 5)];
    }
    bfly(4);
    const __amdgpu_buffer_rsrc_t rd = rsrc(dst + (r < rows ? r : 0) * n + c0);
#pragma unroll
    for (int i = 0; i < 32; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[i]), rd,
                                            r < rows ? (t + 256 * i) * 4 : OOB, 0, 0);
  }
}

// Pure scaling (no transform on this side): dst[r][c] = src[r][c] * rs(r) * cs(c)
__global__ __launch_bounds__(NT) void scale_kernel(const float* __restrict__ src,
                                                   float* __restrict__ dst, int64_t rows,
                                                   int64_t n, Scale rs, Scale cs) {
  const int64_t i4 = ((int64_t)blockIdx.x * NT + threadIdx.x) * 4;
  if (i4 >= rows * n) return;
  const int64_t r = i4 / n, c = i4 % n;
  const float a = scale_at(rs, r);
  float4 q = *(const float4*)(src + i4);
  q.x *= a * scale_at(cs, c);
  q.y *= a * scale_at(cs, c + 1);
  q.z *= a * scale_at(cs, c + 2);
  q.w *= a * scale_at(cs, c + 3);
  *(float4*)(dst + i4) = q;
}

// ---------------------------------------------------------------------------
// column pass: FWHT along the row index over bits [k0, k0 + MB)
// ---------------------------------------------------------------------------
constexpr int CW = 64;       // columns per tile
constexpr int CLD = CW + 4;  // LDS row stride (floats)

template <int MB>
__global__ __launch_bounds__(NT) void col_fwht_kernel(float* __restrict__ M, int64_t rows,
                                                      int64_t ncols, int k0) {
  constexpr int R = 1 << MB;
  constexpr int RA = R >= 16 ? R / 16 : 1;   // rows per thread in phase A (stride 16)
  constexpr int GA = R >= 16 ? 16 : R;       // row groups in phase A
  constexpr int RB = R >= 16 ? 16 : R;       // rows per thread in phase B (consecutive)
  constexpr int GB = R >= 16 ? R / 16 : 1;   // row groups in phase B
  __shared__ __attribute__((aligned(16))) float tile[R * CLD];

  const int64_t beta = blockIdx.x;
  const int64_t base = ((beta >> k0) << (k0 + MB)) | (beta & (((int64_t)1 << k0) - 1));
  const int64_t c = (int64_t)blockIdx.y * CW + 4 * (threadIdx.x & 15);
  const int cq = threadIdx.x & 15;
  const int rg = threadIdx.x >> 4;
  const bool cok = c < ncols;

  // phase A: rows rg + 16*i (i = register index), butterflies over the i bits
  if (rg < GA) {
    float4 v[RA];
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int tr = rg + GA * i;
      const int64_t gr = base + ((int64_t)tr << k0);
      v[i] = cok ? *(const float4*)(M + gr * ncols + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int m = 1; m < RA; m <<= 1)
#pragma unroll
      for (int i = 0; i < RA; ++i) {
        if (i & m) continue;
        const float4 a = v[i], b = v[i | m];
        v[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        v[i | m] = make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
      }
#pragma unroll
    for (int i = 0; i < RA; ++i) *(float4*)(tile + (rg + GA * i) * CLD + 4 * cq) = v[i];
  }
  __syncthreads();
  // phase B: rows RB*rg + i, butterflies over the low bits
  if (rg < GB) {
    float4 v[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) v[i] = *(const float4*)(tile + (RB * rg + i) * CLD + 4 * cq);
#pragma unroll
    for (int m = 1; m < RB; m <<= 1)
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (i & m) continue;
        const float4 a = v[i], b = v[i | m];
        v[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        v[i | m] = make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
      }
    if (cok) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int64_t gr = base + ((int64_t)(RB * rg + i) << k0);
        *(float4*)(M + gr * ncols + c) = v[i];
      }
    }
  }
}

// Column pass for 4096-row blocks in one pass: a workgroup holds a whole block of rows for 8
// columns (128 KB of LDS) and runs all 12 butterfly stages on it, as three rounds of 4 index
// bits in registers (16 rows x 4 columns per thread) with two LDS regroupings, the same rounds
// as the 4096-point row pass:
//   round A: x = 16 t + i      (a thread's 16 rows are consecutive; global loads)
//   round B: x = (t & 15) + 16 i + 256 (t >> 4)
//   round C: x = t + 256 i     (global stores)
// Thread (t, h) = (tid >> 1, tid & 1) owns columns 4h .. 4h + 3 of the slab, so a lane pair
// reads or writes the slab's 32 contiguous bytes of a row.  The four slabs that share a
// 128-byte line of a row run side by side on one XCD (consecutive slabs go to the same XCD),
// so the line is fetched from memory once.  LDS holds (row, column quad) as 16-byte units,
// unit 2x + h XOR-swizzled by ((x >> 4) & 7) << 1: every group of 16 lanes of each round
// touches 16 distinct units modulo 16, i.e. distinct banks.
constexpr int C4K = 4096;
constexpr int C4W = 8;         // columns per workgroup
constexpr int C4T = 512;       // threads
__device__ __forceinline__ int c4_unit(int x, int h) { return (2 * x + h) ^ (((x >> 4) & 7) << 1); }

__global__ __launch_bounds__(C4T) void col_fwht4096_kernel(float* __restrict__ M, int64_t ncols,
                                                            int64_t slabs, int64_t total,
                                                            int64_t per_xcd, int xcds) {
  __shared__ __attribute__((aligned(16))) float4 sm[C4K * C4W / 4];
  const int tid = threadIdx.x, h = tid & 1, t = tid >> 1;
  // workgroup u runs on XCD u mod xcds; XCD x takes items x * per_xcd .. + per_xcd - 1 of the
  // (block, slab) items (the grid is xcds * per_xcd), so neighbouring slabs run side by side
  // on one XCD
  const int64_t u = blockIdx.x;
  const int64_t item = (u % xcds) * per_xcd + u / xcds;
  if (item >= total) return;
  const int64_t blk = item / slabs, slab = item % slabs;
  const int64_t c = slab * C4W + 4 * h;
  const bool cok = c < ncols;
  // descriptor at the block's first row; masked columns read 0 and drop their stores
  const __amdgpu_buffer_rsrc_t rr = rsrc(M + blk * C4K * ncols);
  float4 v[16];
  auto bfly = [&]() {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e & m) continue;
        const float4 a = v[e], b = v[e | m];
        v[e] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        v[e | m] = make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
      }
  };
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = 16 * t + i;
    const int off = cok ? (int)(((int64_t)x * ncols + c) * 4) : OOB;
    const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0);
    v[i] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                       __uint_as_float(q.w));
  }
  bfly();
#pragma unroll
  for (int i = 0; i < 16; ++i) sm[c4_unit(16 * t + i, h)] = v[i];
  __syncthreads();
  const int xb = (t & 15) + 256 * (t >> 4);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = sm[c4_unit(xb + 16 * i, h)];
  bfly();
#pragma unroll
  for (int i = 0; i < 16; ++i) sm[c4_unit(xb + 16 * i, h)] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = sm[c4_unit(t + 256 * i, h)];
  bfly();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = t + 256 * i;
    const int off = cok ? (int)(((int64_t)x * ncols + c) * 4) : OOB;
    const u32x4 q = {__float_as_uint(v[i].x), __float_as_uint(v[i].y), __float_as_uint(v[i].z),
                     __float_as_uint(v[i].w)};
    __builtin_amdgcn_raw_buffer_store_b128(q, rr, off, 0, 0);
  }
}

kq_status launch_col_pass(float* M, int64_t rows, int64_t ncols, int k0, int mb, hipStream_t s) {
  dim3 grid((unsigned)(rows >> mb), (unsigned)ceil_div(ncols, CW));
  switch (mb) {
#define KQ_COL_CASE(X) \
  case X: col_fwht_kernel<X><<<grid, dim3(NT), 0, s>>>(M, rows, ncols, k0); break;
    KQ_COL_CASE(1) KQ_COL_CASE(2) KQ_COL_CASE(3) KQ_COL_CASE(4)
    KQ_COL_CASE(5) KQ_COL_CASE(6) KQ_COL_CASE(7) KQ_COL_CASE(8)
#undef KQ_COL_CASE
    default: return fail(KQ_EINVAL, "column pass width %d", mb);
  }
  KQ_LAUNCHED("col_fwht_kernel");
  return KQ_OK;
}

// FWHT of every column over blocks of b rows (b a power of 2): one pass for 4096-row blocks
// (when a block's byte offsets fit a buffer descriptor), else ceil(log2 b / 8) passes.
kq_status column_transform(float* M, int64_t rows, int64_t ncols, int64_t b, hipStream_t s) {
  if (b == C4K && (int64_t)C4K * ncols * 4 < ((int64_t)1 << 31)) {
    const int64_t slabs = ceil_div(ncols, C4W);
    const int64_t total = (rows / C4K) * slabs;
    if (total > 0x7FFFFFFF) return fail(KQ_ESHAPE, "column pass: too many slabs");
    const int xcds = device_cu_count() % 8 == 0 ? 8 : 1;
    const int64_t per_xcd = ceil_div(total, xcds);
    col_fwht4096_kernel<<<dim3((unsigned)(per_xcd * xcds)), dim3(C4T), 0, s>>>(M, ncols, slabs,
                                                                               total, per_xcd, xcds);
    KQ_LAUNCHED("col_fwht4096_kernel");
    return KQ_OK;
  }
  int m = 0;
  while (((int64_t)1 << m) < b) ++m;
  if (m == 0) return KQ_OK;
  const int passes = (m + 7) / 8;
  int k0 = 0;
  for (int p = 0; p < passes; ++p) {
    const int mb = (m - k0) / (passes - p);
    KQ_TRY(launch_col_pass(M, rows, ncols, k0, mb, s));
    k0 += mb;
  }
  return KQ_OK;
}

// Row transform with fused scaling: every row of dst = FWHT_b(row of src * rs * cs).
kq_status row_transform(const float* src, float* dst, int64_t rows, int64_t n, int64_t b,
                        Scale rs, Scale cs, hipStream_t s) {
  if (b <= 1) {
    const int64_t tot4 = rows * n / 4;
    scale_kernel<<<dim3((unsigned)ceil_div(tot4, NT)), dim3(NT), 0, s>>>(src, dst, rows, n, rs, cs);
    KQ_LAUNCHED("scale_kernel");
    return KQ_OK;
  }
  if (b == RB) {
    // rows per workgroup: all of a workgroup's loads are in flight at once, four rows (64 KB)
    // at most; about four workgroups per CU on a 256-CU device
    const int64_t nb = n / RB;
    const int64_t rpw = (rows * nb) / 1024;
    const int R = rpw >= 4 ? 4 : rpw >= 2 ? 2 : 1;
    const dim3 grid((unsigned)(nb * ceil_div(rows, R)));
    switch (R) {
#define KQ_R4096(X) \
  case X: row_fwht4096_kernel<X><<<grid, dim3(NT), 0, s>>>(src, dst, rows, n, rs, cs); break;
      KQ_R4096(1) KQ_R4096(2) KQ_R4096(4)
#undef KQ_R4096
    }
    KQ_LAUNCHED("row_fwht4096_kernel");
    return KQ_OK;
  }
  if (b == RB8) {
    // two rows per workgroup when that still leaves about four workgroups per CU (four rows
    // per workgroup, two workgroups per CU, ran 3 % slower)
    const int64_t nb = n / RB8;
    const int R = (rows * nb) / 2048 >= 1 ? 2 : 1;
    const dim3 grid((unsigned)(nb * ceil_div(rows, R)));
    if (R == 2) row_fwht8192_kernel<2><<<grid, dim3(NT), 0, s>>>(src, dst, rows, n, rs, cs);
    else row_fwht8192_kernel<1><<<grid, dim3(NT), 0, s>>>(src, dst, rows, n, rs, cs);
    KQ_LAUNCHED("row_fwht8192_kernel");
    return KQ_OK;
  }
  // 16 values per thread up to 1024-point blocks (at most 64 threads, one wave, per block)
  const int ept = b <= 16 ? (int)b : b <= 1024 ? 16 : (int)(b / 256);
  const int tpr = (int)(b / ept);
  const int bpw = NT / tpr;
  const int64_t nblocks = rows * (n / b);
  const dim3 grid((unsigned)ceil_div(nblocks, bpw));
  const size_t shm = tpr > 64 ? (size_t)bpw * b * sizeof(float) : 0;
  switch (ept) {
#define KQ_ROW_CASE(X)                                                                   \
  case X:                                                                                \
    row_fwht_kernel<X><<<grid, dim3(NT), shm, s>>>(src, dst, rows, n, (int)b, rs, cs); \
    break;
    KQ_ROW_CASE(4) KQ_ROW_CASE(8) KQ_ROW_CASE(16) KQ_ROW_CASE(32)
#undef KQ_ROW_CASE
    default: return fail(KQ_EINVAL, "row transform block %lld", (long long)b);
  }
  KQ_LAUNCHED("row_fwht_kernel");
  return KQ_OK;
}

kq_status copy_if_needed(const float* src, float* dst, int64_t count, hipStream_t s) {
  if (src == dst || count == 0) return KQ_OK;
  KQ_HIP(hipMemcpyAsync(dst, src, count * sizeof(float), hipMemcpyDeviceToDevice, s));
  return KQ_OK;
}

bool valid_block(int64_t n, int64_t b) {
  if (b == 1) return true;
  return b >= 4 && b <= 8192 && is_pow2(b) && n % b == 0;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_biip_rotate(const float* W_src, float* W_dst, int64_t out, int64_t in,
                                    const float* HX_src, float* HX_dst, const float* HG_src,
                                    float* HG_dst, const int8_t* sign_in, const int8_t* sign_out,
                                    int64_t had_block_in, int64_t had_block_out, float alpha,
                                    int mode, float* d_in, float* d_out, void* stream) {
  using namespace kq;
  if (mode < KQ_BIIP_FULL || mode > KQ_BIIP_OUT_ONLY)
    return fail(KQ_EINVAL, "kq_biip_rotate: bad mode %d", mode);
  const bool do_in = mode != KQ_BIIP_OUT_ONLY;
  const bool do_out = mode != KQ_BIIP_IN_ONLY;
  const bool rescale = mode != KQ_BIIP_NO_RESCALE;
  if (!W_src || !W_dst || !HX_src || !HX_dst || !d_in || !d_out)
    return fail(KQ_EINVAL, "kq_biip_rotate: NULL argument");
  if ((HG_src == nullptr) != (HG_dst == nullptr))
    return fail(KQ_EINVAL, "kq_biip_rotate: HG_src and HG_dst must both be set or both NULL");
  if (!HG_src && mode != KQ_BIIP_IN_ONLY)
    return fail(KQ_EINVAL, "kq_biip_rotate: H_G is required unless mode is IN_ONLY");
  if ((do_in && !sign_in) || (do_out && !sign_out))
    return fail(KQ_EINVAL, "kq_biip_rotate: sign vector missing");
  if (out < 1 || in < 1 || out % 4 || in % 4 || out > (1 << 30) || in > (1 << 30))
    return fail(KQ_ESHAPE, "kq_biip_rotate: out and in must be positive multiples of 4");
  if (!(alpha >= 0.f) || !isfinite(alpha)) return fail(KQ_EINVAL, "kq_biip_rotate: alpha");
  const int64_t bin = had_block_in == 0 ? (in & -in) : had_block_in;
  const int64_t bout = had_block_out == 0 ? (out & -out) : had_block_out;
  if ((do_in && had_block_in == 0 && bin > 8192) || (do_out && had_block_out == 0 && bout > 8192))
    return fail(KQ_ENOTIMPL,
                "kq_biip_rotate: the automatic Hadamard block (the largest power of 2 dividing the "
                "size) exceeds 8192, the largest block implemented; pass a block of at most 8192");
  if (do_in && !valid_block(in, bin))
    return fail(KQ_ESHAPE, "kq_biip_rotate: input Hadamard block %lld does not tile in=%lld",
                (long long)bin, (long long)in);
  if (do_out && !valid_block(out, bout))
    return fail(KQ_ESHAPE, "kq_biip_rotate: output Hadamard block %lld does not tile out=%lld",
                (long long)bout, (long long)out);
  hipStream_t s = as_stream(stream);

  // 1. rescale vectors (norms of the original W, diagonals of the raw factors)
  // both norm vectors from one read of the original W
  const bool want_col = rescale && do_in, want_row = rescale && do_out;
  if (want_col) KQ_TRY(fill_f32(d_in, in, 0.f, s));
  if (want_col || want_row)
    KQ_TRY(squared_norms(W_src, out, in, want_col ? d_in : nullptr, want_row ? d_out : nullptr, s));
  if (want_col) {
    rescale_kernel<<<dim3((unsigned)ceil_div(in, 256)), dim3(256), 0, s>>>(HX_src, in, d_in, alpha);
    KQ_LAUNCHED("rescale_kernel");
  } else {
    KQ_TRY(fill_f32(d_in, in, 1.f, s));
  }
  if (want_row) {
    rescale_kernel<<<dim3((unsigned)ceil_div(out, 256)), dim3(256), 0, s>>>(HG_src, out, d_out, alpha);
    KQ_LAUNCHED("rescale_kernel");
  } else {
    KQ_TRY(fill_f32(d_out, out, 1.f, s));
  }

  const float isb_in = do_in ? (float)(1.0 / sqrt((double)bin)) : 1.f;
  const float isb_out = do_out ? (float)(1.0 / sqrt((double)bout)) : 1.f;
  // 2. W~ = P_out D_out W D_in P_in^T : fused scaling + row FWHT, then column FWHT
  Scale w_rs{do_out ? d_out : nullptr, do_out ? sign_out : nullptr, 0, isb_out};
  Scale w_cs{do_in ? d_in : nullptr, do_in ? sign_in : nullptr, 0, isb_in};
  KQ_TRY(row_transform(W_src, W_dst, out, in, do_in ? bin : 1, w_rs, w_cs, s));
  if (do_out) KQ_TRY(column_transform(W_dst, out, in, bout, s));
  // 3. H~_X = P_in D_in^-1 H_X D_in^-1 P_in^T
  if (do_in) {
    Scale hs{d_in, sign_in, 1, isb_in};
    KQ_TRY(row_transform(HX_src, HX_dst, in, in, bin, hs, hs, s));
    KQ_TRY(column_transform(HX_dst, in, in, bin, s));
  } else {
    KQ_TRY(copy_if_needed(HX_src, HX_dst, in * in, s));
  }
  // 4. H~_G = P_out D_out^-1 H_G D_out^-1 P_out^T
  if (HG_src) {
    if (do_out) {
      Scale hs{d_out, sign_out, 1, isb_out};
      KQ_TRY(row_transform(HG_src, HG_dst, out, out, bout, hs, hs, s));
      KQ_TRY(column_transform(HG_dst, out, out, bout, s));
    } else {
      KQ_TRY(copy_if_needed(HG_src, HG_dst, out * out, s));
    }
  }
  return KQ_OK;
}
