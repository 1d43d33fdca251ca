// Two-sided rounding: GPTQ on vec(W) under the Kronecker Hessian
//   H_d = (H_X + lam_X I) (x) (H_G + lam_G I),  U = chol_upper(H_d^-1) = U_X (x) U_G.
//
// BaKron abstract (the two-sided adaptive-rounding formulation of BoA and YAQA, computed
// in O(m + n) sequential steps with O(mn(m + n)) work).  With c = i m + r the position of
// W[r, i] in vec(W), coordinate c is rounded with q = code(w_c), e = (w_c - qhat_c) / U[c, c]
// and feeds w_c' -= e U[c, c'].  U[(i, r), (i', r')] = U_X[i, i'] U_G[r, r'] vanishes unless
// i' >= i and r' >= r, so a coordinate depends only on those above and to its left, and all
// coordinates of one anti-diagonal r + i can be rounded together.
//
// Schedule: 32 x 32 tiles and, per anti-diagonal of tiles, two launches.  F = E U_X (E the
// scaled errors, zero until a tile has run) collects each finished tile's errors pushed to
// the right.  For every tile (R, I) of the diagonal:
//   1. pull: the pending feedback sum_{R'' <= R} U_G[R'', R]^T F[R'', I] (every tile above
//      or to the left is done), split over slices of 256 contraction indices, one workgroup
//      each (fp32 MFMA), partial sums kept per slice and added in a fixed order;
//   2. round: one workgroup per tile rounds its 63 anti-diagonals; each step's errors e_k
//      (one per row) feed the whole tile through U_G[k, r'] U_X[d - k, i'], a 32 x 32 x 32
//      product of which each wave forms and applies one 16 x 16 quadrant (LDS float atomics,
//      or partials summed across waves, cost several times the whole loop here).  The
//      workgroup then pushes its errors into its own and the next column block,
//      F[R, I..I+1] += E_tile U_X[I, I..I+1], with operands loaded before the rounding;
//   3. push: the rest, F[R, I+2..] += E_tile U_X[I, I+2..], split over chunks of 256
//      columns (fp32 MFMA).  Nothing before diagonal d + 2 reads those columns, so these
//      workgroups share a launch with the pull of the next diagonal.
// Pulls cost O(m^2 n) and pushes O(m n^2) in all, as in the BaKron bound.
//
// Grids: per (row, group) asymmetric min-max from W~ before rounding (a static grid; every
// dependency-respecting order then gives the same codes), groups of whole tiles.  Scales in
// fp32 from an fp64 division, zero points in fp64 as the oracle takes them.
#include "kq_internal.h"

#include <math.h>

#include <algorithm>

namespace kq {
namespace {

constexpr int TS = 32;   // tile edge

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KS = 256;  // contraction indices per pull slice
constexpr int PS = 256;  // columns per push chunk
constexpr int MAXSL = 16;  // pull slices summed per batch of loads in the round kernel

struct TSArgs {
  const float* W;        // m x n, ld n (W~)
  const float* UX;       // n x n, ld n, explicit upper inverse factor
  const float* UG;       // m x m, ld m
  const float* scale;    // m x ng
  const uint8_t* zero;   // m x ng
  const uint8_t* deadX;  // n: zero column of W
  const uint8_t* deadG;  // m: zero row of W
  float* F;              // m x n, E U_X of the finished tiles
  float* E;              // m x n, scaled errors
  float* part;           // pull partial sums: [tile of the diagonal][slice][32 x 32]
  uint8_t* codes;        // m x n
  int m, n, ng, group, maxq;
  int d;                 // tile anti-diagonal
  int r_lo;              // its first tile row
  int nslice;            // slices per tile in part (the most any tile of a diagonal needs)
};

__device__ __forceinline__ int acc_row(int r, int kh) { return 8 * (r >> 2) + 4 * kh + (r & 3); }

// 1. pull, slice s of tile (R, I): sum over k in [s KS, min(32 (R + 1), (s + 1) KS)) of
//    U_G[k][r0 + r'] F[k][c0 + i'].  The four waves take interleaved k pairs, 16 pairs' loads
//    in flight before their products.
__device__ __forceinline__ void ts_pull(const TSArgs& a, int b, float (*red)[TS * TS]) {
  const int tix = b / a.nslice, sl = b % a.nslice;
  const int R = a.r_lo + tix, I = a.d - R;
  const int r0 = TS * R, c0 = TS * I;
  const int K = r0 + TS, kb = sl * KS, ke = min(K, kb + KS);
  if (kb >= ke) return;
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  const int wave = t >> 6;
  const int64_t n = a.n, m = a.m;
  f32x16 acc = f32x16{};
  // pairs k0 = kb + 2 (wave + 4 j), j = 0 .. (ke - kb) / 8 - 1 (ke - kb is a multiple of 32)
  const int npairs = (ke - kb) / 8;
  for (int j0 = 0; j0 < npairs; j0 += 16) {
    float av[16], bv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int k = kb + 2 * (wave + 4 * min(j0 + j, npairs - 1)) + kh;
      av[j] = a.UG[(int64_t)k * m + r0 + l32];
      bv[j] = a.F[(int64_t)k * n + c0 + l32];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j0 + j < npairs) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][acc_row(r, kh) * TS + l32] = acc[r];
  __syncthreads();
  float* out = a.part + ((int64_t)tix * a.nslice + sl) * (TS * TS);
  for (int e = t; e < TS * TS; e += 256) out[e] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
}

// 2. round tile (R, I): W~ (dead rows / columns zero) minus the pulled feedback, then the
//    tile's own anti-diagonals; then its errors pushed into its own and the next column block.
__global__ __launch_bounds__(256) void ts_round_kernel(TSArgs a) {
  __shared__ float wt[TS][TS + 1];    // the tile's weights minus the pulled feedback
  __shared__ float ugd[TS][TS + 1];   // U_G diagonal block [k][r']
  __shared__ float uxd[TS][TS + 1];   // U_X diagonal block [i][i']
  __shared__ float et[TS][TS + 1];    // scaled errors
  __shared__ uint8_t ct[TS][TS];      // codes
  __shared__ float ed[TS];            // errors of the current in-tile anti-diagonal, by row
  __shared__ float srow[TS], zrow[TS], sinv[TS];
  __shared__ float rug[TS], rux[TS];  // 1 / U_G[r][r], 1 / U_X[i][i] of the tile's rows, columns
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int tix = blockIdx.x;
  const int R = a.r_lo + tix, I = a.d - R;
  const int r0 = TS * R, c0 = TS * I;
  const int64_t n = a.n, m = a.m;
  const int nsl = (r0 + TS + KS - 1) / KS;   // slices this tile's pull used
  const int g = c0 / a.group;                // groups hold whole tiles
  {
    // the slices' partial sums through a descriptor bounded to them: every load issued at
    // once, the ones past the last slice read 0
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (int64_t)tix * a.nslice * (TS * TS), 0, nsl * TS * TS * 4, 0x00020000);
    float ps[4][MAXSL];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int sl = 0; sl < MAXSL; ++sl)
        ps[q][sl] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rp, 4 * (sl * TS * TS + t + 256 * q), 0, 0));
    for (int sl0 = MAXSL; sl0 < nsl; sl0 += MAXSL)   // tiles below row 2^12 / 32: more slices
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int sl = 0; sl < MAXSL; ++sl)
          ps[q][sl] += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rp, 4 * ((sl0 + sl) * TS * TS + t + 256 * q), 0, 0));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = t + 256 * q, r = e >> 5, c = e & 31;
      ugd[r][c] = a.UG[(int64_t)(r0 + r) * m + r0 + c];
      uxd[r][c] = a.UX[(int64_t)(c0 + r) * n + c0 + c];
      const bool dead = a.deadG[r0 + r] || a.deadX[c0 + c];
      float w = dead ? 0.f : a.W[(int64_t)(r0 + r) * n + c0 + c];
#pragma unroll
      for (int sl = 0; sl < MAXSL; ++sl) w -= ps[q][sl];
      wt[r][c] = w;
    }
  }
  if (t < TS) {
    const float sc = a.scale[(int64_t)(r0 + t) * a.ng + g];
    srow[t] = sc;
    sinv[t] = 1.0f / sc;
    zrow[t] = (float)a.zero[(int64_t)(r0 + t) * a.ng + g];
  }
  __syncthreads();
  if (t < TS) {
    rug[t] = 1.0f / ugd[t][t];
    rux[t] = 1.0f / uxd[t][t];
  }
  __syncthreads();

  // operands of the near push (F[R, I..I+1] and U_X[I, I+1]), loaded now so that their
  // latency passes under the rounding: no other workgroup of this launch writes them
  const bool near = wave == 0 || (wave == 1 && c0 + TS < a.n);
  const int cbn = c0 + TS * (wave & 1);
  float nbv[16], nfo[16];
  if (near) {
#pragma unroll
    for (int j = 0; j < 16; ++j) nbv[j] = a.UX[(int64_t)(c0 + 2 * j + kh) * n + cbn + l32];
#pragma unroll
    for (int r = 0; r < 16; ++r) nfo[r] = a.F[(int64_t)(r0 + acc_row(r, kh)) * n + cbn + l32];
  }

  // Wave w owns the 16 x 16 quadrant (rows 16 (w >> 1), columns 16 (w & 1)) of each step's
  // feedback Delta[r'][i'] = sum_k U_G[k][r'] e_k U_X[dd - k][i'] (v_mfma_f32_16x16x4f32, k in
  // fours): A[r'][kk] = U_G[k][r'] is fixed, B[kk][i'] = e_k U_X[dd - k][i'].
  const int q0 = 16 * (wave >> 1), q1 = 16 * (wave & 1), l16 = lane & 15, kq = lane >> 4;
  float aop[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) aop[j] = ugd[4 * j + kq][q0 + l16];
  for (int dd = 0; dd < 2 * TS - 1; ++dd) {
    if (t < TS) {
      const int i = dd - t;
      float e = 0.f;
      if (i >= 0 && i < TS) {
        const float w = wt[t][i], s = srow[t], z = zrow[t];
        const float q = fminf(fmaxf(rintf(w * sinv[t]) + z, 0.f), (float)a.maxq);
        const float qh = s * (q - z);
        e = (w - qh) * (rug[t] * rux[i]);
        et[t][i] = e;
        ct[t][i] = (uint8_t)q;
      }
      ed[t] = e;
    }
    __syncthreads();
    // k-blocks with a coordinate on the diagonal: 4 j + 3 >= dd - 31 and 4 j <= dd; only rows
    // k <= r' reach the quadrant (U_G upper), so blocks past its last row add nothing
    const int jlo = max(0, (dd - (TS - 1)) >> 2), jhi = min(min(7, dd >> 2), (q0 + 15) >> 2);
    if (jlo <= jhi) {
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < jlo || j > jhi) continue;   // uniform
        const int k = 4 * j + kq, ii = dd - k;
        const float bv = (ii >= 0 && ii < TS) ? ed[k] * uxd[ii < 0 ? 0 : (ii >= TS ? TS - 1 : ii)][q1 + l16] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[j], bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) wt[q0 + 4 * kq + j][q1 + l16] -= acc[j];
    }
    __syncthreads();
  }
  // near push: F[R, I] += E_tile U_X[I, I] (wave 0) and F[R, I + 1] += E_tile U_X[I, I + 1]
  // (wave 1), the products in the order the far push takes for the other blocks
  if (near) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(et[l32][2 * j + kh], nbv[j], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) a.F[(int64_t)(r0 + acc_row(r, kh)) * n + cbn + l32] = nfo[r] + acc[r];
  }
  // errors and codes out once the tile is done (a global store inside the loop would make
  // every barrier wait for it)
  for (int e = t; e < TS * TS; e += 256) {
    const int r = e >> 5, c = e & 31;
    a.E[(int64_t)(r0 + r) * n + c0 + c] = et[r][c];
    a.codes[(int64_t)(r0 + r) * n + c0 + c] = ct[r][c];
  }
}

// 3. far push, chunk c of tile (R, I): F[r0 + r][col] += sum_k E[r0 + r][c0 + k] U_X[c0 + k][col]
//    for the chunk's columns (at or right of c0 + 64), 32 per wave block.
__device__ __forceinline__ void ts_push_far(const TSArgs& a, int b, int nchunk) {
  const int tix = b / nchunk, ch = b % nchunk;
  const int R = a.r_lo + tix, I = a.d - R;
  const int r0 = TS * R, c0 = TS * I;
  const int cb0 = c0 + 2 * TS + ch * PS;
  if (cb0 >= a.n) return;
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, kh = lane >> 5;
  const int wave = t >> 6;
  const int64_t n = a.n;
  float eop[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) eop[j] = a.E[(int64_t)(r0 + l32) * n + c0 + 2 * j + kh];
  const int nblk = min(PS, a.n - cb0) / TS;
  for (int blk = wave; blk < nblk; blk += 4) {
    const int cb = cb0 + TS * blk;
    float bv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) bv[j] = a.UX[(int64_t)(c0 + 2 * j + kh) * n + cb + l32];
    float fo[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) fo[r] = a.F[(int64_t)(r0 + acc_row(r, kh)) * n + cb + l32];
    f32x16 acc = f32x16{};
#pragma unroll
    for (int j = 0; j < 16; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(eop[j], bv[j], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) a.F[(int64_t)(r0 + acc_row(r, kh)) * n + cb + l32] = fo[r] + acc[r];
  }
}

// One launch: the pull workgroups of diagonal d + 1 (ap, npull of them) and the far-push
// workgroups of diagonal d (aq, nchunk per tile).  The two sets touch disjoint data: the pull
// reads F's column blocks I of its tiles, which the far push of diagonal d does not write.
__global__ __launch_bounds__(256) void ts_pull_push_kernel(TSArgs ap, int npull, TSArgs aq, int nchunk) {
  __shared__ float red[4][TS * TS];
  const int b = blockIdx.x;
  if (b < npull) ts_pull(ap, b, red);
  else ts_push_far(aq, b - npull, nchunk);
}

// Static grid per (row, group) from W~ with dead rows and columns zeroed: one wave each.
// xmin = min(0, min), xmax = max(0, max), s = (xmax - xmin) / maxq (1 when equal),
// z = rint(-xmin / s); s and z in fp64, s stored as fp32.
__global__ __launch_bounds__(256) void ts_grid_kernel(const float* __restrict__ W, int64_t m, int64_t n,
                                                      int group, int maxq, const uint8_t* __restrict__ deadX,
                                                      const uint8_t* __restrict__ deadG,
                                                      float* __restrict__ scale, uint8_t* __restrict__ zero) {
  const int64_t ng = n / group;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= m * ng) return;
  const int64_t r = item / ng, g = item % ng;
  const int lane = threadIdx.x & 63;
  float lo = 0.f, hi = 0.f;
  if (!deadG[r]) {
    for (int64_t c = g * group + lane; c < (g + 1) * group; c += 64) {
      const float w = deadX[c] ? 0.f : W[r * n + c];
      lo = fminf(lo, w);
      hi = fmaxf(hi, w);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if (lane == 0) {
    double s = ((double)hi - (double)lo) / (double)maxq;
    if (hi == lo) s = 1.0;
    const double z = rint(-(double)lo / s);
    scale[item] = (float)s;
    zero[item] = (uint8_t)z;
  }
}

// Packed words: bit k of row r's stream is bit (k mod bits) of code floor(k / bits).
__global__ __launch_bounds__(256) void ts_pack_kernel(const uint8_t* __restrict__ codes, int64_t m,
                                                      int64_t n, int bits, uint32_t* __restrict__ packed) {
  const int64_t wpr = n * bits / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= m * wpr) return;
  const int64_t r = idx / wpr, wd = idx % wpr;
  uint32_t v = 0;
  for (int b = 0; b < 32; ++b) {
    const int64_t k = 32 * wd + b;
    v |= (uint32_t)((codes[r * n + k / bits] >> (k % bits)) & 1u) << b;
  }
  packed[idx] = v;
}

struct TSWorkspace {
  float* UX;
  float* UG;
  float* Ffac;   // factorization scratch: kmax^2
  float* Tsc;    // 128 kmax
  float* F;      // m x n
  float* E;      // m x n
  float* part;   // pull partial sums
  uint8_t* codes;
  uint8_t* deadX;
  uint8_t* deadG;
  double* lam;
  int* flag;
};

int64_t ts_layout(int64_t m, int64_t n, char* base, TSWorkspace* w) {
  const int64_t k = std::max(m, n);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += (bytes + 255) / 256 * 256;
    return base ? base + o : nullptr;
  };
  TSWorkspace x;
  x.UX = (float*)take(n * n * 4);
  x.UG = (float*)take(m * m * 4);
  x.Ffac = (float*)take(k * k * 4);
  x.Tsc = (float*)take(128 * k * 4);
  x.F = (float*)take(m * n * 4);
  x.E = (float*)take(m * n * 4);
  x.part = (float*)take(std::min(m, n) / TS * (m / KS + 1) * TS * TS * 4);
  x.codes = (uint8_t*)take(m * n);
  x.deadX = (uint8_t*)take(n);
  x.deadG = (uint8_t*)take(m);
  x.lam = (double*)take(8);
  x.flag = (int*)take(4);
  if (w) *w = x;
  return off;
}

kq_status ts_check(const kq_quant_params* p, int64_t out, int64_t in) {
  if (!p) return fail(KQ_EINVAL, "kq_quantize_two_sided: params is NULL");
  if (p->bits < 2 || p->bits > 4) return fail(KQ_EINVAL, "kq_quantize_two_sided: bits must be 2, 3 or 4");
  if (p->asym != 1) return fail(KQ_ENOTIMPL, "kq_quantize_two_sided: only the asymmetric grid (asym = 1)");
  if (p->act_order != 0 || p->w_clip != 0)
    return fail(KQ_ENOTIMPL, "kq_quantize_two_sided: act_order and w_clip are not implemented");
  if (!(p->damp >= 0.0f)) return fail(KQ_EINVAL, "kq_quantize_two_sided: damp must be >= 0");
  if (out < 128 || in < 128 || out % 128 != 0 || in % 128 != 0 || out > 32768 || in > 32768)
    return fail(KQ_ESHAPE, "kq_quantize_two_sided: out and in must be multiples of 128 (<= 32768)");
  if (p->group < TS || p->group % TS != 0 || in % p->group != 0)
    return fail(KQ_ESHAPE, "kq_quantize_two_sided: group must be a multiple of 32 dividing in");
  if ((in * p->bits) % 32 != 0) return fail(KQ_ESHAPE, "kq_quantize_two_sided: in * bits %% 32 != 0");
  return KQ_OK;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_quantize_two_sided_workspace(const kq_quant_params* p, int64_t out,
                                                     int64_t in, size_t* bytes) {
  using namespace kq;
  if (!bytes) return fail(KQ_EINVAL, "kq_quantize_two_sided_workspace: bytes is NULL");
  KQ_TRY(ts_check(p, out, in));
  *bytes = (size_t)ts_layout(out, in, nullptr, nullptr);
  return KQ_OK;
}

extern "C" kq_status kq_quantize_two_sided(const kq_quant_params* p, const float* W, const float* HX,
                                           const float* HG, int64_t out, int64_t in, uint32_t* packed,
                                           float* scales, uint8_t* zeros, void* ws, size_t ws_bytes,
                                           uint8_t* codes_opt, void* stream) {
  using namespace kq;
  KQ_TRY(ts_check(p, out, in));
  if (!W || !HX || !HG || !packed || !scales || !zeros || !ws)
    return fail(KQ_EINVAL, "kq_quantize_two_sided: NULL argument");
  const size_t need = (size_t)ts_layout(out, in, nullptr, nullptr);
  if (ws_bytes < need) return fail(KQ_EWORKSPACE, "kq_quantize_two_sided: workspace of %zu bytes needed", need);
  TSWorkspace w;
  ts_layout(out, in, (char*)ws, &w);
  hipStream_t s = as_stream(stream);
  const int64_t m = out, n = in;
  KQ_HIP(hipMemsetAsync(w.flag, 0, sizeof(int), s));
  KQ_TRY(explicit_inverse_factor(HX, n, p->damp, w.Ffac, w.Tsc, w.deadX, w.lam, w.flag, w.UX, s));
  KQ_TRY(explicit_inverse_factor(HG, m, p->damp, w.Ffac, w.Tsc, w.deadG, w.lam, w.flag, w.UG, s));
  const int maxq = (1 << p->bits) - 1;
  const int64_t items = m * (n / p->group);
  ts_grid_kernel<<<dim3((unsigned)ceil_div(items, 4)), dim3(256), 0, s>>>(W, m, n, p->group, maxq, w.deadX,
                                                                         w.deadG, scales, zeros);
  KQ_LAUNCHED("ts_grid_kernel");
  KQ_TRY(fill_f32(w.F, m * n, 0.0f, s));
  uint8_t* codes = codes_opt ? codes_opt : w.codes;
  TSArgs a;
  a.W = W; a.UX = w.UX; a.UG = w.UG; a.scale = scales; a.zero = zeros;
  a.deadX = w.deadX; a.deadG = w.deadG; a.F = w.F; a.E = w.E; a.part = w.part; a.codes = codes;
  a.m = (int)m; a.n = (int)n; a.ng = (int)(n / p->group); a.group = p->group; a.maxq = maxq;
  const int NR = (int)(m / TS), NI = (int)(n / TS), ND = NR + NI - 1;
  // the tiles of diagonal d: rows r_lo .. r_hi; the lowest one pulls the most slices
  auto diagonal = [&](int d, TSArgs& x) {
    x = a;
    x.d = d;
    x.r_lo = std::max(0, d - (NI - 1));
    const int r_hi = std::min(d, NR - 1);
    x.nslice = (TS * (r_hi + 1) + KS - 1) / KS;
    return r_hi - x.r_lo + 1;
  };
  TSArgs ap;
  const int t0 = diagonal(0, ap);
  ts_pull_push_kernel<<<dim3((unsigned)(t0 * ap.nslice)), dim3(256), 0, s>>>(ap, t0 * ap.nslice, ap, 0);
  KQ_LAUNCHED("ts_pull_push_kernel");
  for (int d = 0; d < ND; ++d) {
    TSArgs ar;
    const int tiles = diagonal(d, ar);
    ts_round_kernel<<<dim3((unsigned)tiles), dim3(256), 0, s>>>(ar);
    KQ_LAUNCHED("ts_round_kernel");
    // the pulls of diagonal d + 1 and the far pushes of diagonal d in one launch; the
    // leftmost tile of d pushes the most columns
    TSArgs an = ar;
    const int npull = d + 1 < ND ? diagonal(d + 1, an) * an.nslice : 0;
    const int I_lo = d - (ar.r_lo + tiles - 1);
    const int64_t far_cols = n - (int64_t)TS * (I_lo + 2);
    const int nchunk = far_cols > 0 ? (int)ceil_div(far_cols, PS) : 0;
    const int64_t total = (int64_t)npull + (int64_t)tiles * nchunk;
    if (total > 0) {
      ts_pull_push_kernel<<<dim3((unsigned)total), dim3(256), 0, s>>>(an, npull, ar, nchunk);
      KQ_LAUNCHED("ts_pull_push_kernel");
    }
  }
  const int64_t words = m * (n * p->bits / 32);
  ts_pack_kernel<<<dim3((unsigned)ceil_div(words, 256)), dim3(256), 0, s>>>(codes, m, n, p->bits, packed);
  KQ_LAUNCHED("ts_pack_kernel");
  int flag = 0;
  KQ_HIP(hipMemcpyAsync(&flag, w.flag, sizeof(int), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  if (flag) return fail(KQ_ENOTSPD, "kq_quantize_two_sided: a damped factor has no Cholesky factor");
  return KQ_OK;
}
