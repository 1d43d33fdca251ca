// Hessian factor H = A^T A (or H += A^T A) from a token-major bf16 stream.
//
// KronQ README, opening section: the layer Hessian is approximated as
// H_X (x) H_G, with H_X built from calibration activations and H_G from
// output gradients (WaterKron and FlipFlop Hessian, Table 1, "Marginal":
// E[x x^T] and E[g g^T]).  Both are the same operation on different streams.
//
// Two kernels compute the same H; the direct-to-LDS one is the default.
//
// Direct-to-LDS kernel (syrk_dma_kernel):
//   * 256 x 256 output tiles over the lower block triangle, 4 waves of 64; each wave owns a
//     128 x 128 sub-tile = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (fp32 accumulators in
//     AGPRs; bf16 products are exact in fp32).
//   * The stream is copied into LDS token-major, as it lies in memory, by the load unit
//     itself (global_load_lds, 16 bytes per lane): no registers are spent on staging, and a
//     ring of four 32-token stages (128 KB) keeps three stages of copies in flight.  The
//     MFMA operands (8 consecutive tokens of one channel per lane) are read with the
//     transposing LDS read ds_read_b64_tr_b16; a per-token-row XOR swizzle of the 16-byte
//     chunks keeps those reads free of bank conflicts.
//   * Each wave copies the same number of chunks in every stage (tokens outside the split
//     read a 16-byte zero chunk), so the per-stage vmcnt waits are exact; one workgroup
//     barrier per stage hands buffers over.  Operand reads, copies and MFMAs are interleaved
//     explicitly, operands in the order the MFMAs consume them.
//   * XCD-aware order: workgroup u runs on XCD u mod 8; each XCD walks a contiguous region
//     of tiles split by split, so the tiles resident on one XCD share panels in its L2 and
//     all XCDs stream the same token range at the same time (last-level cache reuse).  The
//     token split count is the smallest that fills whole rounds of an XCD's CUs.
//   * Partial tiles are added to H with fp32 atomics (H is zeroed first unless
//     accumulating); a final pass mirrors the lower triangle into the upper one.
//
// Register-staged kernel (syrk_bf16_kernel): 64-token stages loaded into registers as 8
// tokens x 4 channels per thread, transposed in registers and stored channel-major into two
// LDS buffers with an XOR-permuted chunk layout; 4 or 8 waves; split-major or tile-major
// order.  It serves strides too large for the direct kernel's 32-bit per-stage offsets.
#include "device_util.h"
#include "kq_internal.h"

namespace kq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TILE = 256;          // output tile edge (channels)
constexpr int BK = 64;             // tokens per stage
constexpr int PANEL = TILE * BK;   // bf16 elements of one panel in LDS (no padding)
constexpr int BAND = 4;            // tile rows per band in the visiting order

struct SyrkArgs {
  const uint16_t* A;   // the tiles' row channels
  int64_t lda;
  const uint16_t* B;   // the tiles' column channels (B == A for a Hessian; only the
  int64_t ldb;         // direct-to-LDS kernel reads B)
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

// Register-staged kernel.
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

// ---------------------------------------------------------------------------------------------
// Direct-to-LDS variant.  The stream is copied into LDS token-major, exactly as it lies in
// memory, by the load unit itself (global_load_lds, 16 bytes per lane, 1 KB per wave
// instruction): no registers are spent on staging and up to four 32-token stages are in
// flight at once.  The MFMA operands, which need 8 consecutive tokens of one channel per lane,
// are then read with the transposing LDS read ds_read_b64_tr_b16: within each 16-lane group,
// lane 4e+q points at token e, channels 4q..4q+3, and lane i receives channel i, tokens 0..3.
// A token row holds the tile's 256 channels as 32 chunks of 16 bytes; chunk k of token t is
// stored in slot k ^ swz(t mod 4) with swz = {0, 10, 6, 12}, which puts the four token rows
// read by each half-wave (and by each quarter-wave) on disjoint banks.
// ---------------------------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int DBK = 32;                  // tokens per stage
constexpr int DPANEL = DBK * TILE;       // bf16 elements of one panel (16 KB)
constexpr int DSTAGE = 2 * DPANEL;       // both panels of a stage (32 KB)
constexpr int DWAVES = 4;
constexpr int DMA_PER_PANEL = DPANEL * 2 / 1024 / DWAVES;   // 1 KB wave instructions per wave

__device__ __forceinline__ int dswz(int e) { return (0xC6A0 >> (4 * e)) & 15; }

// Sixteen zero bytes in device memory: the source of every copy lane whose token lies outside
// the split, so that each wave issues the same number of copies in every stage and the
// vmcnt-based waits stay exact.
__device__ __attribute__((aligned(16))) uint32_t g_zero_chunk[4];

// Copy tokens [t0, t0 + DBK) x channels [cbase, cbase + 256) of the stream into a panel.
// Wave w fills 1 KB blocks DMA_PER_PANEL*w + r (two token rows each); lane l of a block
// writes slot l & 31 of token row 2p + (l >> 5).  off[r] is the lane's element offset from
// the stage's first token row (row * lda + channel; channels at or beyond n are read from
// channel 0 of the same token, their products only reach entries of H outside the matrix).
// dma_sources computes the lane's source addresses, dma_copy issues the copies.
__device__ __forceinline__ void dma_sources(const uint16_t* __restrict__ base, int64_t t0,
                                            int64_t tend, const uint32_t (&off)[DMA_PER_PANEL],
                                            int wave, int lane,
                                            const uint16_t* (&src)[DMA_PER_PANEL]) {
  const uint16_t* zero = (const uint16_t*)g_zero_chunk;
#pragma unroll
  for (int r = 0; r < DMA_PER_PANEL; ++r) {
    const int row = 2 * (DMA_PER_PANEL * wave + r) + (lane >> 5);
    src[r] = t0 + row < tend ? base + off[r] : zero;
  }
}

__device__ __forceinline__ void dma_copy(const uint16_t* const (&src)[DMA_PER_PANEL],
                                         uint16_t* panel, int wave) {
#pragma unroll
  for (int r = 0; r < DMA_PER_PANEL; ++r)
    __builtin_amdgcn_global_load_lds(
        (const void*)src[r],
        (__attribute__((address_space(3))) void*)(panel + (DMA_PER_PANEL * wave + r) * 512), 16,
        0, 0);
}

__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* p) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p + 4 * TILE));
  const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

struct DmaArgs {
  SyrkArgs s;
  int per_xcd;      // tiles per XCD region
  int xcds;
};

// DNST = stages in the LDS ring (128 KB); each buffer is its own LDS object so that the
// compiler can tell the reads of one stage from the copies into another.
constexpr int DNST = 4;
__global__ __launch_bounds__(DWAVES * 64) void syrk_dma_kernel(DmaArgs d) {
  const SyrkArgs& a = d.s;
  __shared__ __attribute__((aligned(1024))) uint16_t b0[DSTAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[DSTAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t b2[DSTAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t b3[DSTAGE];

  // workgroup u runs on XCD u mod xcds; each XCD walks its own contiguous region of tiles,
  // split by split, so the tiles resident on one XCD share panels in its L2 and all XCDs
  // stream the same token range at the same time
  const int u = blockIdx.x;
  const int xcd = u % d.xcds;
  const int q = u / d.xcds;
  const int split = q / d.per_xcd;
  const int tile = xcd * d.per_xcd + q % d.per_xcd;
  if (tile >= a.ntiles || split >= a.splits) return;
  int bi, bj;
  tile_of(tile, a.nb, bi, bj);
  const int64_t tbeg = (int64_t)split * a.tok_split;
  const int64_t tend = min(a.T, tbeg + a.tok_split);
  if (tbeg >= tend) return;
  const int nst_real = (int)((tend - tbeg + DBK - 1) / DBK);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int ci = bi * TILE, cj = bj * TILE;

  // stage-invariant part of this lane's copy sources (see dma_panel)
  uint32_t offi[DMA_PER_PANEL], offj[DMA_PER_PANEL];
#pragma unroll
  for (int r = 0; r < DMA_PER_PANEL; ++r) {
    const int row = 2 * (DMA_PER_PANEL * wave + r) + (lane >> 5);
    const int k8 = 8 * ((lane & 31) ^ dswz(row & 3));
    offi[r] = (uint32_t)(row * a.lda) + (uint32_t)(ci + k8 < a.n ? ci + k8 : 0);
    offj[r] = (uint32_t)(row * a.ldb) + (uint32_t)(cj + k8 < a.n ? cj + k8 : 0);
  }

  // per-lane element offsets of the operand reads inside a panel (first token half, kk = 0)
  const int e = (lane >> 2) & 3, qq = lane & 3, g = lane >> 4;
  const int rowoff = (8 * (g >> 1) + e) * TILE + 4 * (qq & 1);
  int offA[4], offB[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    offA[m] = rowoff + 8 * ((4 * m + 2 * (g & 1) + (qq >> 1)) ^ dswz(e)) + 128 * wr;
    offB[m] = rowoff + 8 * ((4 * m + 2 * (g & 1) + (qq >> 1)) ^ dswz(e)) + 128 * wc;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[m][k] = f32x16{};

  // Stages at or beyond the split's end (the ring runs DNST stages ahead) copy zeros.
  // Diagonal tiles copy their one panel twice, which keeps every tile on one code path.
  const uint16_t* srci[DMA_PER_PANEL];
  const uint16_t* srcj[DMA_PER_PANEL];
  auto sources = [&](int s) {
    const int64_t t0 = tbeg + (int64_t)s * DBK;
    dma_sources(a.A + min(t0, tend) * a.lda, t0, tend, offi, wave, lane, srci);
    dma_sources(a.B + min(t0, tend) * a.ldb, t0, tend, offj, wave, lane, srcj);
  };
  auto issue = [&](uint16_t* buf) {
    dma_copy(srci, buf, wave);
    dma_copy(srcj, buf + DPANEL, wave);
  };
  // operands are read in the order the multiplies consume them: a0, b0..b3, a1..a3
  auto read = [&](const uint16_t* buf, int kk, bf16x8 (&av)[4], bf16x8 (&bv)[4]) {
    const uint16_t* pi = buf + kk * 16 * TILE;
    const uint16_t* pj = buf + DPANEL + kk * 16 * TILE;
    av[0] = tr_operand(pi + offA[0]);
#pragma unroll
    for (int k = 0; k < 4; ++k) bv[k] = tr_operand(pj + offB[k]);
#pragma unroll
    for (int m = 1; m < 4; ++m) av[m] = tr_operand(pi + offA[m]);
  };
  auto mma = [&](const bf16x8 (&av)[4], const bf16x8 (&bv)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        acc[m][k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bv[k], acc[m][k], 0, 0, 0);
  };
  // wait until this wave's copies of stage s+1 have landed: every stage issues the same number
  // of copies and stages up to s + DNST - 1 have been issued
  auto wait_next = [&]() { __builtin_amdgcn_s_waitcnt(wait_vm(2 * DMA_PER_PANEL * (DNST - 2))); };

  // The stage count is rounded up to whole rounds of the ring; stages past the split's end
  // are copied as zeros and add nothing.  Every stage of a round then uses a fixed buffer.
  const int nst = ((nst_real + DNST - 1) / DNST) * DNST;
  bf16x8 xa[4], xb[4], ya[4], yb[4];
  sources(0); issue(b0);
  sources(1); issue(b1);
  sources(2); issue(b2);
  sources(3); issue(b3);
  __builtin_amdgcn_s_waitcnt(wait_vm(2 * DMA_PER_PANEL * (DNST - 1)));
  lds_barrier();
  read(b0, 0, xa, xb);

  // Stage s: operands of its first 16 tokens are already in registers (xa, xb).  Read the
  // second 16 (ya, yb) early while multiplying the first, and prepare the copy sources of
  // stage s + DNST; wait for this wave's copies of stage s+1 and for every wave's reads of
  // stage s; refill stage s's buffer with stage s + DNST and read the first operands of
  // stage s+1 while multiplying the second half of stage s.  (After the last stage the read
  // of the next buffer is harmless and unused.)
#define KQ_DMA_STEP(J, CUR, NXT)                                   \
  {                                                                \
    const int s = s0 + (J);                                        \
    read(CUR, 1, ya, yb);                                          \
    mma(xa, xb);                                                   \
    sources(s + DNST);                                             \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);           \
    }                                                              \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);             \
    __builtin_amdgcn_sched_barrier(0);                             \
    wait_next();                                                   \
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);                        \
    lds_barrier();                                                 \
    issue(CUR);                                                    \
    read(NXT, 0, xa, xb);                                          \
    mma(ya, yb);                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);           \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);           \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);           \
    }                                                              \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);             \
    __builtin_amdgcn_sched_barrier(0);                             \
  }
  for (int s0 = 0; s0 < nst; s0 += DNST) {
    KQ_DMA_STEP(0, b0, b1)
    KQ_DMA_STEP(1, b1, b2)
    KQ_DMA_STEP(2, b2, b3)
    KQ_DMA_STEP(3, b3, b0)
  }
#undef KQ_DMA_STEP
  // the ring's trailing copies (zeros) must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // epilogue: lane holds column l32 of each 32x32 block; rows 8*(r/4) + 4*(lane/32) + r%4
  const int l32 = lane & 31, rh = (lane >> 5) * 4;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int gj = cj + 128 * wc + 32 * k + l32;
      if (gj >= a.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gi = ci + 128 * wr + 32 * m + 8 * (r >> 2) + rh + (r & 3);
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

// H[i][j] = H[j][i] for i < j, in 64 x 64 tiles through LDS.  A thread's 16 loads are issued
// before any is used: indices are clamped into the matrix (a branch around a load would make
// the compiler wait for it), and only entries inside the matrix are stored.
__global__ __launch_bounds__(256) void mirror_lower_to_upper(float* __restrict__ H, int64_t ldh,
                                                             int n, int m) {
  __shared__ float t[64][65];
  // upper-triangle tile (ti, tj), ti <= tj, enumerated row by row: rows before ti hold
  // S(ti) = ti (2m - ti + 1) / 2 tiles; ti from the quadratic's root, corrected for rounding
  const int idx = blockIdx.x;
  auto before = [&](int r) { return (int64_t)r * (2 * m - r + 1) / 2; };
  const float bq = 2.0f * (float)m + 1.0f;
  int ti = (int)((bq - sqrtf(fmaxf(bq * bq - 8.0f * (float)idx, 0.0f))) * 0.5f);
  ti = max(0, min(ti, m - 1));
  while (ti > 0 && before(ti) > idx) --ti;
  while (ti + 1 < m && before(ti + 1) <= idx) ++ti;
  const int tj = ti + (int)(idx - before(ti));
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // source tile (tj, ti) of the lower part: rows tj*64.., cols ti*64..
  float v[16];
  const int sj = min(ti * 64 + tx, n - 1);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int si = min(tj * 64 + ty + 4 * k, n - 1);
    v[k] = H[(int64_t)si * ldh + sj];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) t[ty + 4 * k][tx] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = ty + 4 * k;
    const int gi = ti * 64 + r, gj = tj * 64 + tx;  // destination (upper)
    if (gi < n && gj < n && gi < gj) H[(int64_t)gi * ldh + gj] = t[tx][r];
  }
}

// Token splits for the direct-to-LDS kernel: the smallest S (>= 2 stages of work per tile
// each) whose per-XCD workgroup count fills whole rounds of the XCD's CUs to within 3 %, with
// at least two workgroups per CU in all.
int choose_splits_dma(int per_xcd, int cu_per_xcd, int xcds, int64_t T) {
  int64_t max_s = T / (8 * DBK);
  if (max_s < 1) max_s = 1;
  if (max_s > 64) max_s = 64;
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= max_s; ++s) {
    const int64_t items = (int64_t)per_xcd * s;
    const int64_t rounds = (items + cu_per_xcd - 1) / cu_per_xcd;
    const double eff = (double)items / (double)(rounds * cu_per_xcd);
    if (items * xcds < 2LL * cu_per_xcd * xcds) continue;
    if (eff >= 0.97) return s;
    if (eff > best_eff + 1e-9) { best_eff = eff; best = s; }
  }
  return best;
}

// Token splits for the register-staged kernel: at least ~2048 workgroups (8 per CU) for load
// balance, a multiple of 8, at least 8 stages per split.
int choose_splits(int ntiles, int64_t T) {
  int s = 8;
  while ((int64_t)ntiles * s < 2048 && s < 64) s += 8;
  int64_t max_s = T / (8 * BK);
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = (int)max_s;
  return s;
}

}  // namespace

// H's lower block triangle (+)= sum_t A[t, i] B[t, j] (bf16 streams, T tokens, n channels), then
// optionally the mirror of the lower triangle into the upper one.  B == A is the Hessian
// A^T A; a second stream B takes the direct-to-LDS kernel, whose 32-bit stage offsets it
// needs (KQ_ENOTIMPL otherwise).
kq_status gram_lower(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t T,
                     int64_t n, float* H, int64_t ldh, bool accumulate, bool mirror, hipStream_t s) {
  const int ni = (int)n;
  if (!accumulate) {
    zero_lower_tiles<<<dim3(ni), dim3(256), 0, s>>>(H, ldh, ni);
    KQ_LAUNCHED("zero_lower_tiles");
  }
  if (T > 0) {
    SyrkArgs a;
    a.A = A; a.lda = lda; a.B = B; a.ldb = ldb; a.T = T; a.n = ni; a.H = H; a.ldh = ldh;
    a.nb = (int)ceil_div(n, TILE);
    a.ntiles = a.nb * (a.nb + 1) / 2;
    a.splits = choose_splits(a.ntiles, T);
    a.tok_split = ceil_div(ceil_div(T, a.splits), BK) * BK;
    a.splits = (int)ceil_div(T, a.tok_split);
    // the direct-to-LDS kernel (the default) keeps 32-bit per-lane offsets within a 32-token
    // stage; larger strides take the register-staged kernel (so may the engine's tests)
    const bool dma_fits = (int64_t)DBK * std::max(lda, ldb) + n < ((int64_t)1 << 32);
    int variant = B == A ? (int)testing_value(KQ_TESTING_SYRK_KERNEL, 4) : 4;
    if (variant < 0 || variant > 4) variant = 4;
    if (variant == 4 && !dma_fits) {
      if (B != A) return fail(KQ_ENOTIMPL, "two-stream Gram product: stream stride too large");
      variant = 3;
    }
    if (variant == 4) {
      DmaArgs d;
      d.xcds = device_cu_count() % 8 == 0 ? 8 : 1;
      const int cu_per_xcd = device_cu_count() / d.xcds;
      d.per_xcd = (int)ceil_div(a.ntiles, d.xcds);
      a.splits = choose_splits_dma(d.per_xcd, cu_per_xcd, d.xcds, T);
      a.tok_split = ceil_div(ceil_div(T, a.splits), DBK) * DBK;
      a.splits = (int)ceil_div(T, a.tok_split);
      d.s = a;
      const int64_t g = (int64_t)d.xcds * d.per_xcd * a.splits;
      if (g > 0x7FFFFFFF) return fail(KQ_ESHAPE, "kq_accumulate_hessian: too many tiles");
      syrk_dma_kernel<<<dim3((unsigned)g), dim3(DWAVES * 64), 0, s>>>(d);
      KQ_LAUNCHED("syrk_dma_kernel");
    } else {
      const int64_t grid = (int64_t)a.ntiles * a.splits;
      if (grid > 0x7FFFFFFF) return fail(KQ_ESHAPE, "kq_accumulate_hessian: too many tiles");
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
  }
  if (mirror) {
    const int m = (int)ceil_div(n, 64);
    const int64_t mt = (int64_t)m * (m + 1) / 2;
    mirror_lower_to_upper<<<dim3((unsigned)mt), dim3(256), 0, s>>>(H, ldh, ni, m);
    KQ_LAUNCHED("mirror_lower_to_upper");
  }
  return KQ_OK;
}

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
  return gram_lower(A_bf16, lda, A_bf16, lda, T, n, H, ldh, accumulate != 0, true,
                    as_stream(stream));
}
