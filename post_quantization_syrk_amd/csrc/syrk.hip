// Hessian factor H = A^T A (or H += A^T A) from a token-major bf16 stream.
//
// KronQ README, opening section: the layer Hessian is approximated as
// H_X (x) H_G, with H_X built from calibration activations and H_G from
// output gradients (WaterKron and FlipFlop Hessian, Table 1, "Marginal":
// E[x x^T] and E[g g^T]).  Both are the same operation on different streams.
//
// Kernel design (gfx950, CDNA4):
//   * 256 x 256 output tiles over the lower block triangle, 256 threads
//     (4 waves of 64); each wave owns a 128 x 128 sub-tile = 4 x 4 blocks of
//     v_mfma_f32_32x32x16_bf16 (fp32 accumulators, bf16 products are exact),
//     which keeps LDS operand traffic at 8 KB per 16 MFMAs.
//   * The token axis is the reduction axis and is the slow axis of the
//     stream, so every 64-token stage is loaded as 16 tokens x 4 channels per
//     thread (coalesced 512-byte rows per wave), transposed in registers to
//     channel-major order and stored to LDS, where each MFMA operand is one
//     16-byte read of 8 consecutive tokens.  A channel's 64 tokens fill one
//     128-byte LDS row whose eight 16-byte chunks are permuted by
//     chunk ^ ((c ^ (c >> 3)) & 7): both the transposed stores (lanes 4
//     channels apart) and the operand reads (lanes 1 channel apart) then hit
//     distinct banks.
//   * Two LDS buffers: the next stage's global loads are in flight while the
//     current stage runs on the matrix cores.
//   * The token range is split S ways (S a multiple of 8, about 2048
//     workgroups in all).  Workgroups are numbered split-major: the ones
//     dispatched together work on the same token range, so the streamed
//     tokens are shared through the L2s and the last-level cache.  Tiles are
//     visited in bands of 4 tile rows so neighbouring tiles share panels.
//     Partial tiles are added to H with fp32 atomics (H is zeroed first
//     unless accumulating).  Measured on the 4096-wide, 131072-token factor:
//     8 waves per workgroup (2 per SIMD) beat 4 waves (1 per SIMD), and
//     split-major beat tile-major order.
//   * A final pass mirrors the lower triangle into the upper one.
#include "kq_internal.h"

#include <stdlib.h>

namespace kq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TILE = 256;          // output tile edge (channels)
constexpr int BK = 64;             // tokens per stage
constexpr int PANEL = TILE * BK;   // bf16 elements of one panel in LDS (no padding)
constexpr int BAND = 4;            // tile rows per band in the visiting order

struct SyrkArgs {
  const uint16_t* A;
  int64_t lda;
  int64_t T;
  int n;
  float* H;
  int64_t ldh;
  int nb;              // panels = ceil(n / TILE)
  int ntiles;          // nb * (nb + 1) / 2
  int splits;          // token splits
  int64_t tok_split;   // tokens per split (multiple of BK)
};

// Visiting order of the lower block triangle: bands of BAND tile rows; inside
// a band, column-panel major.  Returns (bi, bj) with bi >= bj.
__device__ __forceinline__ void tile_of(int t, int nb, int& bi, int& bj) {
  int band0 = 0;
  for (;;) {
    int r1 = min(band0 + BAND, nb);
    // tiles in this band: sum over rows bi in [band0, r1) of (bi + 1)
    int cnt = (r1 * (r1 + 1) - band0 * (band0 + 1)) / 2;
    if (t < cnt) {
      // columns bj = 0 .. r1-1; column bj holds rows max(bj, band0) .. r1-1
      int bjc = 0;
      for (;;) {
        int rows = r1 - max(bjc, band0);
        if (t < rows) {
          bi = max(bjc, band0) + t;
          bj = bjc;
          return;
        }
        t -= rows;
        ++bjc;
      }
    }
    t -= cnt;
    band0 = r1;
  }
}

// LDS offset (bf16 elements) of the 8-token chunk kc of channel c.
__device__ __forceinline__ int lds_off(int c, int kc) {
  return c * BK + ((kc ^ ((c ^ (c >> 3)) & 7)) << 3);
}

// 8 tokens x 4 channels of bf16 for one thread: r[i] holds token i, channels c..c+3.
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ A, int64_t lda, int64_t t,
                                           int64_t tend, int c, int n, bool full, uint2 (&r)[8]) {
  if (full) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = *(const uint2*)(A + (t + i) * lda + c);
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (t + i < tend) {
      const uint16_t* row = A + (t + i) * lda;
      if (c + 3 < n) {
        uint2 v = *(const uint2*)(row + c);
        w[0] = v.x & 0xFFFFu; w[1] = v.x >> 16; w[2] = v.y & 0xFFFFu; w[3] = v.y >> 16;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c + k < n) w[k] = row[c + k];
      }
    }
    r[i].x = w[0] | (w[1] << 16);
    r[i].y = w[2] | (w[3] << 16);
  }
}

// Store the 8x4 block transposed: channel cl + k gets tokens 8*kc .. 8*kc+7 as one 16-byte
// chunk.  Lanes of odd cl/4 write their channels in the order 1, 0, 3, 2, so the channels
// written by one instruction alternate in parity across lanes (distinct banks).
__device__ __forceinline__ void store_block(uint16_t* __restrict__ panel, int cl, int kc,
                                            const uint2 (&r)[8]) {
  uint4 v0, v1, v2, v3;
  // low / high halves of each 32-bit word are channels c and c+1 (x) or c+2 and c+3 (y)
  v0.x = (r[0].x & 0xFFFFu) | (r[1].x << 16);
  v0.y = (r[2].x & 0xFFFFu) | (r[3].x << 16);
  v0.z = (r[4].x & 0xFFFFu) | (r[5].x << 16);
  v0.w = (r[6].x & 0xFFFFu) | (r[7].x << 16);
  v1.x = (r[0].x >> 16) | (r[1].x & 0xFFFF0000u);
  v1.y = (r[2].x >> 16) | (r[3].x & 0xFFFF0000u);
  v1.z = (r[4].x >> 16) | (r[5].x & 0xFFFF0000u);
  v1.w = (r[6].x >> 16) | (r[7].x & 0xFFFF0000u);
  v2.x = (r[0].y & 0xFFFFu) | (r[1].y << 16);
  v2.y = (r[2].y & 0xFFFFu) | (r[3].y << 16);
  v2.z = (r[4].y & 0xFFFFu) | (r[5].y << 16);
  v2.w = (r[6].y & 0xFFFFu) | (r[7].y << 16);
  v3.x = (r[0].y >> 16) | (r[1].y & 0xFFFF0000u);
  v3.y = (r[2].y >> 16) | (r[3].y & 0xFFFF0000u);
  v3.z = (r[4].y >> 16) | (r[5].y & 0xFFFF0000u);
  v3.w = (r[6].y >> 16) | (r[7].y & 0xFFFF0000u);
  const int o = (cl >> 2) & 1;
  const uint4 w0 = o ? v1 : v0, w1 = o ? v0 : v1, w2 = o ? v3 : v2, w3 = o ? v2 : v3;
  *(uint4*)(panel + lds_off(cl + (0 ^ o), kc)) = w0;
  *(uint4*)(panel + lds_off(cl + (1 ^ o), kc)) = w1;
  *(uint4*)(panel + lds_off(cl + (2 ^ o), kc)) = w2;
  *(uint4*)(panel + lds_off(cl + (3 ^ o), kc)) = w3;
}

// WAVES = 4: 128 x 128 per wave (1 wave per SIMD); WAVES = 8: 128 x 64 per wave (2 per SIMD).
// SPLIT_MAJOR: consecutive workgroups share a token range (all tiles of one split run
// together, so the concurrently streamed tokens stay in the last-level cache);
// otherwise consecutive workgroups share a tile (split = blockIdx % S, one range per XCD).
template <int WAVES, bool SPLIT_MAJOR>
__global__ __launch_bounds__(WAVES * 64) void syrk_bf16_kernel(SyrkArgs a) {
  constexpr int THREADS = WAVES * 64;
  constexpr int TPT = 64 / (THREADS / 64);   // tokens per thread per stage (16 or 8)
  constexpr int WN = WAVES == 4 ? 4 : 2;     // 32-wide column blocks per wave
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * PANEL];

  const int u = blockIdx.x;
  const int split = SPLIT_MAJOR ? u / a.ntiles : u % a.splits;
  const int tile = SPLIT_MAJOR ? u % a.ntiles : u / a.splits;
  int bi, bj;
  tile_of(tile, a.nb, bi, bj);
  const bool diag = (bi == bj);

  const int64_t tbeg = (int64_t)split * a.tok_split;
  const int64_t tend = min(a.T, tbeg + a.tok_split);
  if (tbeg >= tend) return;
  const int nstages = (int)((tend - tbeg + BK - 1) / BK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // loader mapping: TPT tokens (TPT/8 chunks) starting at TPT*tg, channels 4*cg .. 4*cg+3
  const int tg = tid >> 6;
  const int cg = tid & 63;
  const int ci = bi * TILE + 4 * cg;
  const int cj = bj * TILE + 4 * cg;
  const bool full_i = (bi + 1) * TILE <= a.n;
  const bool full_j = (bj + 1) * TILE <= a.n;

  // compute mapping: wave tile rows [128*wr, +128) of panel i, cols [32*WN*wc, +32*WN) of panel j
  const int wr = WAVES == 4 ? (wave >> 1) : (wave >> 2);
  const int wc = WAVES == 4 ? (wave & 1) : (wave & 3);
  const int l32 = lane & 31;
  const int kh = lane >> 5;

  f32x16 acc[4][WN];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int k = 0; k < WN; ++k) acc[m][k] = f32x16{};

  uint2 ri0[8], ri1[8], rj0[8], rj1[8];

#define KQ_SYRK_LOAD(T0)                                                                   \
  {                                                                                        \
    const bool tf = (T0) + BK <= tend;                                                     \
    load_block(a.A, a.lda, (T0) + TPT * tg, tend, ci, a.n, tf && full_i, ri0);             \
    if (TPT == 16) load_block(a.A, a.lda, (T0) + TPT * tg + 8, tend, ci, a.n, tf && full_i, ri1); \
    if (!diag) {                                                                           \
      load_block(a.A, a.lda, (T0) + TPT * tg, tend, cj, a.n, tf && full_j, rj0);           \
      if (TPT == 16) load_block(a.A, a.lda, (T0) + TPT * tg + 8, tend, cj, a.n, tf && full_j, rj1); \
    }                                                                                      \
  }
#define KQ_SYRK_STORE(Q)                                                                   \
  {                                                                                        \
    store_block((Q), 4 * cg, (TPT / 8) * tg, ri0);                                         \
    if (TPT == 16) store_block((Q), 4 * cg, 2 * tg + 1, ri1);                              \
    if (!diag) {                                                                           \
      store_block((Q) + PANEL, 4 * cg, (TPT / 8) * tg, rj0);                               \
      if (TPT == 16) store_block((Q) + PANEL, 4 * cg, 2 * tg + 1, rj1);                    \
    }                                                                                      \
  }

  KQ_SYRK_LOAD(tbeg)
  KQ_SYRK_STORE(lds)
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    const uint16_t* pi = lds + buf * 2 * PANEL;
    const uint16_t* pj = diag ? pi : pi + PANEL;
    const bool more = s + 1 < nstages;
    if (more) KQ_SYRK_LOAD(tbeg + (int64_t)(s + 1) * BK)
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = 2 * ks + kh;
      bf16x8 av[4], bv[WN];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        av[m] = *(const bf16x8*)(pi + lds_off(128 * wr + 32 * m + l32, kc));
#pragma unroll
      for (int k = 0; k < WN; ++k)
        bv[k] = *(const bf16x8*)(pj + lds_off(32 * WN * wc + 32 * k + l32, kc));
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int k = 0; k < WN; ++k)
          acc[m][k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bv[k], acc[m][k], 0, 0, 0);
    }
    if (more) KQ_SYRK_STORE(lds + (buf ^ 1) * 2 * PANEL)
    __syncthreads();
  }
#undef KQ_SYRK_LOAD
#undef KQ_SYRK_STORE

  // epilogue: lane holds column l32 of each 32x32 block; rows 8*(r/4) + 4*(lane/32) + r%4
  const int rh = kh * 4;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int k = 0; k < WN; ++k) {
      const int gj = bj * TILE + 32 * WN * wc + 32 * k + l32;
      if (gj >= a.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gi = bi * TILE + 128 * wr + 32 * m + 8 * (r >> 2) + rh + (r & 3);
        if (gi < a.n) atomicAdd(a.H + (int64_t)gi * a.ldh + gj, acc[m][k][r]);
      }
    }
  }
}

// Zero the lower block triangle of H (the region the tiles add into).
__global__ void zero_lower_tiles(float* __restrict__ H, int64_t ldh, int n) {
  const int row = blockIdx.x;
  const int cend = min(n, (row / TILE + 1) * TILE);
  float* p = H + (int64_t)row * ldh;
  for (int c = threadIdx.x; c < cend; c += blockDim.x) p[c] = 0.0f;
}

// H[i][j] = H[j][i] for i < j, in 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void mirror_lower_to_upper(float* __restrict__ H, int64_t ldh,
                                                             int n, int m) {
  __shared__ float t[64][65];
  // upper-triangle tile (ti, tj), ti <= tj, enumerated row by row
  int idx = blockIdx.x, ti = 0;
  while (idx >= m - ti) { idx -= m - ti; ++ti; }
  const int tj = ti + idx;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // read source tile (tj, ti) of the lower part: rows tj*64.., cols ti*64..
  for (int r = ty; r < 64; r += 4) {
    const int gi = tj * 64 + r, gj = ti * 64 + tx;
    if (gi < n && gj < n) t[r][tx] = H[(int64_t)gi * ldh + gj];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int gi = ti * 64 + r, gj = tj * 64 + tx;  // destination (upper)
    if (gi < n && gj < n && gi < gj) H[(int64_t)gi * ldh + gj] = t[tx][r];
  }
}

// Kernel variant: bit 0 = 8 waves (else 4), bit 1 = split-major order.  KQ_SYRK_VARIANT
// overrides the default (a tuning knob; every variant computes the same H).
int syrk_variant() {
  const char* env = getenv("KQ_SYRK_VARIANT");
  if (env) {
    const int v = atoi(env);
    if (v >= 0 && v <= 3) return v;
  }
  return 3;
}

int choose_splits(int ntiles, int64_t T) {
  const char* env = getenv("KQ_SYRK_SPLITS");
  if (env) {
    int v = atoi(env);
    if (v >= 1) return v;
  }
  // at least ~2048 workgroups (8 per CU) for load balance, a multiple of 8, at least 8
  int s = 8;
  while ((int64_t)ntiles * s < 2048 && s < 64) s += 8;
  // keep at least 8 stages per split
  int64_t max_s = T / (8 * BK);
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = (int)max_s;
  return s;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_accumulate_hessian(const uint16_t* A_bf16, int64_t T, int64_t n,
                                           int64_t lda, float* H, int64_t ldh, int accumulate,
                                           void* stream) {
  using namespace kq;
  if (!H) return fail(KQ_EINVAL, "kq_accumulate_hessian: H is NULL");
  if (T < 0 || n < 1 || n > (int64_t)1 << 30)
    return fail(KQ_ESHAPE, "kq_accumulate_hessian: bad sizes T=%lld n=%lld", (long long)T,
                (long long)n);
  if (T > 0 && !A_bf16) return fail(KQ_EINVAL, "kq_accumulate_hessian: A is NULL");
  if (lda < n || lda % 8 != 0)
    return fail(KQ_ESHAPE, "kq_accumulate_hessian: lda=%lld must be >= n and a multiple of 8",
                (long long)lda);
  if (ldh < n) return fail(KQ_ESHAPE, "kq_accumulate_hessian: ldh < n");
  if (((uintptr_t)A_bf16) % 16 != 0)
    return fail(KQ_EINVAL, "kq_accumulate_hessian: A must be 16-byte aligned");
  if (accumulate != 0 && accumulate != 1)
    return fail(KQ_EINVAL, "kq_accumulate_hessian: accumulate must be 0 or 1");
  hipStream_t s = as_stream(stream);
  const int ni = (int)n;
  if (!accumulate) {
    zero_lower_tiles<<<dim3(ni), dim3(256), 0, s>>>(H, ldh, ni);
    KQ_LAUNCHED("zero_lower_tiles");
  }
  if (T > 0) {
    SyrkArgs a;
    a.A = A_bf16; a.lda = lda; a.T = T; a.n = ni; a.H = H; a.ldh = ldh;
    a.nb = (int)ceil_div(n, TILE);
    a.ntiles = a.nb * (a.nb + 1) / 2;
    a.splits = choose_splits(a.ntiles, T);
    a.tok_split = ceil_div(ceil_div(T, a.splits), BK) * BK;
    a.splits = (int)ceil_div(T, a.tok_split);
    const int64_t grid = (int64_t)a.ntiles * a.splits;
    if (grid > 0x7FFFFFFF) return fail(KQ_ESHAPE, "kq_accumulate_hessian: too many tiles");
    const int variant = syrk_variant();
    const bool split_major = (variant & 2) != 0;
    if (variant & 1) {
      if (split_major) syrk_bf16_kernel<8, true><<<dim3((unsigned)grid), dim3(512), 0, s>>>(a);
      else syrk_bf16_kernel<8, false><<<dim3((unsigned)grid), dim3(512), 0, s>>>(a);
    } else {
      if (split_major) syrk_bf16_kernel<4, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
      else syrk_bf16_kernel<4, false><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
    }
    KQ_LAUNCHED("syrk_bf16_kernel");
  }
  const int m = (int)ceil_div(n, 64);
  const int64_t mt = (int64_t)m * (m + 1) / 2;
  mirror_lower_to_upper<<<dim3((unsigned)mt), dim3(256), 0, s>>>(H, ldh, ni, m);
  KQ_LAUNCHED("mirror_lower_to_upper");
  return KQ_OK;
}
