// Deploy side: one BiIP-quantized layer applied to an activation vector (batch 1),
//   y = D_out^-1 P_out^T Qhat P_in D_in^-1 x,   Qhat[r, c] = s[r, g] (q[r, c] - z[r, g]).
//
// KronQ README, opening section: the packed int4/int2 weights are dequantized on the fly by a
// fused dequant + BiIP matvec for single-token decode.  Here:
//   * matvec kernel: each workgroup owns 16 rows (4 per wave) and first issues the loads of
//     its rows' packed words (16 bytes per lane, a row's words contiguous across the wave's
//     lanes), scales and zero points;
//   * while they are in flight it forms x~ = Had_b(S_in . x / d_in) / sqrt(b) in LDS (every
//     workgroup for itself): each thread loads 16 contiguous entries and takes the first four
//     butterfly stages in registers, the remaining stages go in radix-16 rounds through LDS;
//   * a lane's codes are unpacked byte-wise (v_cvt_f32_ubyte) and a row's dot product is taken
//     as s (sum q x~ - z sum x~) per chunk, the x~ values read once for the wave's 4 rows;
//   * output blocks of at most 16 rows are rotated by the workgroup that owns them; larger
//     ones need rows of many workgroups, so the matvec kernel writes y~ = Qhat x~ to y and a
//     second kernel rotates and rescales y in place (one workgroup per 4096 entries or per
//     block).  The kernel boundary orders the two: no device-wide fence inside a kernel, which
//     on this chip writes back and invalidates the whole L2 of the workgroup's XCD.
// At full rate the layer is HBM-bound: out * in * bits / 8 bytes of packed words per call.
#include "device_util.h"
#include "kq_internal.h"

#include <math.h>

#include <string.h>

#include <algorithm>

namespace kq {
namespace {

constexpr int DT = 256;     // threads per workgroup
constexpr int DR = 16;      // output blocks up to this many rows are rotated in the matvec kernel
constexpr int SEG = 4096;   // entries per workgroup of the output rotation (or one block)

constexpr int MAXL = 8;     // layers per grouped call

// One layer of a call (all layers of a call read the same x).
struct LayerArgs {
  const uint32_t* packed;  // out x wpr words
  const float* scales;     // out x ngroups
  const uint8_t* zeros;    // out x ngroups
  const float* d_in;
  const float* d_out;
  const int8_t* s_in;
  const int8_t* s_out;
  float* y;
  int out, wpr, ngroups, bits;
  int bin, bout;
  float isb_in, isb_out;   // 1 / sqrt(block)
  unsigned gmagic;         // ceil(2^32 / group): c / group = umulhi(c, gmagic) for c < 2^16
  int wg0;                 // first matvec workgroup of the layer
  int seg, sg0;            // output rotation: entries per workgroup, first workgroup
};

struct GroupArgs {
  LayerArgs L[MAXL];
  const float* x;
  int nl, in, xlen;        // layers; x entries; LDS length of x~ (whole chunks)
};

// The layer of workgroup `wg` given ascending first workgroups (empty ranges allowed).
__device__ __forceinline__ int layer_of(const GroupArgs& a, int wg, bool outrot) {
  int l = 0;
  for (int k = 1; k < a.nl; ++k)
    if (wg >= (outrot ? a.L[k].sg0 : a.L[k].wg0)) l = k;
  return l;
}

// LDS index of entry i: 16 floats of padding after every 256 entries, so that the strided
// accesses of the radix-16 rounds spread over the banks; runs of 16 stay contiguous and
// 16-byte aligned.
__device__ __forceinline__ int pad(int i) { return i + ((i >> 8) << 4); }
__host__ __device__ constexpr int padded_len(int n) { return n + (((n + 255) >> 8) << 4); }

// Butterfly stages of strides 1, 2, .., R/2 on r[0..N) (unnormalized, Sylvester order):
// the R-point transform of every R-run of r[0..N).
template <int R, int N = R>
__device__ __forceinline__ void bfly(float (&r)[16]) {
#pragma unroll
  for (int s = 1; s < R; s <<= 1)
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((j & s) == 0) {
        const float a = r[j], c = r[j | s];
        r[j] = a + c;
        r[j | s] = a - c;
      }
}

// The R-point transforms (R = 1, 2, 4, 8 or 16) of the 16 / R runs of r.
__device__ __forceinline__ void bfly_runs16(float (&r)[16], int R) {
  switch (R) {
    case 16: bfly<16, 16>(r); break;
    case 8: bfly<8, 16>(r); break;
    case 4: bfly<4, 16>(r); break;
    case 2: bfly<2, 16>(r); break;
    default: break;
  }
}

// One radix-R round over v (LDS, padded) of n entries: the stages of strides h .. h R / 2.
template <int R>
__device__ __forceinline__ void lds_round(float* v, int n, int h, int lh) {
  for (int p = threadIdx.x; p < n / R; p += DT) {
    const int base = (((p >> lh) * R) << lh) | (p & (h - 1));
    float r[16];
#pragma unroll
    for (int j = 0; j < R; ++j) r[j] = v[pad(base + j * h)];
    bfly<R>(r);
#pragma unroll
    for (int j = 0; j < R; ++j) v[pad(base + j * h)] = r[j];
  }
}

// Stages of strides 16 .. b/2 of the b-block Walsh-Hadamard transform of v[0..n) in LDS,
// after the thread-local stages of strides 1 .. 8 (all threads; a barrier after each round).
__device__ __forceinline__ void lds_fwht_rest(float* v, int n, int b) {
  for (int h = 16; h < b; h <<= 4) {
    const int R = b / h >= 16 ? 16 : b / h, lh = __builtin_ctz(h);
    switch (R) {
      case 16: lds_round<16>(v, n, h, lh); break;
      case 8: lds_round<8>(v, n, h, lh); break;
      case 4: lds_round<4>(v, n, h, lh); break;
      default: lds_round<2>(v, n, h, lh); break;
    }
    __syncthreads();
  }
}

// mul * sign / d from a loaded d word and the word holding the sign byte (an absent d reads
// 0 and counts as 1; an absent sign reads 0, i.e. +1).  v_rcp_f32: 1 ulp.
__device__ __forceinline__ float factor(unsigned dw, unsigned sw, int byte, bool hd, float mul) {
  const float d = hd ? __uint_as_float(dw) : 1.f;
  const float f = mul * __builtin_amdgcn_rcpf(d);
  return ((sw >> (8 * byte + 7)) & 1u) ? -f : f;
}

// f[j] = mul * sign[c + j] / d[c + j] for j < 16 (an absent vector counts as 1); d and sg
// hold n entries and are uniform across the workgroup.
__device__ __forceinline__ void factors16(const float* d, const int8_t* sg, float mul, int c,
                                          int n, float (&f)[16]) {
  const bool hd = d != nullptr, hs = sg != nullptr;
  const __amdgpu_buffer_rsrc_t rd = rsrc(d, hd ? 4 * n : 0), rg = rsrc(sg, hs ? n : 0);
  u32x4 dv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) dv[q] = __builtin_amdgcn_raw_buffer_load_b128(rd, 4 * (c + 4 * q), 0, 0);
  const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rg, c, 0, 0);
#pragma unroll
  for (int j = 0; j < 16; ++j) f[j] = factor(dv[j >> 2][j & 3], sv[j >> 2], j & 3, hd, mul);
}

// Loads of B groups of 16 entries per thread (groups g0 + DT k): src entries and, when the
// input factors are applied, d and the signs; groups at or past n read zero.
template <int B>
struct StageRegs {
  u32x4 xv[B][4];
  u32x4 dv[B][4];
  u32x4 sv[B];
};

template <int B>
__device__ __forceinline__ void stage_load(StageRegs<B>& S, const __amdgpu_buffer_rsrc_t rs,
                                           const __amdgpu_buffer_rsrc_t rd,
                                           const __amdgpu_buffer_rsrc_t rg, bool pre, int g0) {
#pragma unroll
  for (int k = 0; k < B; ++k) {
    const int c = 16 * (g0 + DT * k);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      S.xv[k][q] = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (c + 4 * q), 0, 0);
      if (pre) S.dv[k][q] = __builtin_amdgcn_raw_buffer_load_b128(rd, 4 * (c + 4 * q), 0, 0);
    }
    if (pre) S.sv[k] = __builtin_amdgcn_raw_buffer_load_b128(rg, c, 0, 0);
  }
}

// v (LDS, padded) <- the loaded groups below len, times mul * sign / d when `pre` (zero at or
// past n), with their thread-local butterfly stages (R-point runs).
template <int B, bool GUARD>
__device__ __forceinline__ void stage_finish(float* v, const StageRegs<B>& S, bool hd, bool pre,
                                             float mul, int n, int len, int R, int g0) {
#pragma unroll
  for (int k = 0; k < B; ++k) {
    const int c = 16 * (g0 + DT * k);
    if (GUARD && c >= len) break;
    const bool ok = c < n;
    float r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float xj = __uint_as_float(S.xv[k][j >> 2][j & 3]);
      if (pre) {
        const float f = factor(S.dv[k][j >> 2][j & 3], S.sv[k][j >> 2], j & 3, hd, mul);
        r[j] = ok ? xj * f : 0.f;
      } else {
        r[j] = xj;
      }
    }
    bfly_runs16(r, R);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(v + pad(c + 4 * q)) = make_float4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
  }
}

// v (LDS, padded) <- the b-block transform of src[0..n) (times mul * sign / d when `pre`),
// entries n .. len zero.  n and len are multiples of 16; src, d, sg uniform across the
// workgroup.  `between` runs after the first batch of loads is issued and before any of
// them is used (it issues other loads that then overlap the transform).  The first batch is
// written whole, so v holds at least 16 * DT * B entries (beyond len: zeros); an unguarded
// first batch keeps its loads ahead of `between` (a guard would let the compiler sink them
// into the guarded block, after the other loads).
template <int B, typename F>
__device__ __forceinline__ void stage_rotated(float* v, const float* src, const float* d,
                                              const int8_t* sg, float mul, bool pre, int n,
                                              int len, int b, F between) {
  const bool hd = d != nullptr, hs = sg != nullptr;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src, 4 * n), rd = rsrc(d, pre && hd ? 4 * n : 0),
                               rg = rsrc(sg, pre && hs ? n : 0);
  const int R = b >= 16 ? 16 : b, ng = len / 16, t = threadIdx.x;
  {
    StageRegs<B> S;
    stage_load<B>(S, rs, rd, rg, pre, t);
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
    stage_finish<B, false>(v, S, hd, pre, mul, n, len, R, t);
  }
  for (int g0 = t + B * DT; g0 < ng; g0 += B * DT) {
    StageRegs<B> S;
    stage_load<B>(S, rs, rd, rg, pre, g0);
    stage_finish<B, true>(v, S, hd, pre, mul, n, len, R, g0);
  }
  __syncthreads();
  lds_fwht_rest(v, n, b);
}

// Rows [rw0, rw0 + 4 RPW) of layer L (RPW rows per wave): y~ (or y, when its output blocks
// fit in 16 rows).
template <int BITS, int MC, int B, int RPW>
__device__ __forceinline__ void matvec_rows(const GroupArgs& a, const LayerArgs& L, int rw0,
                                            float* xs) {
  constexpr int CPW = 32 / BITS;        // codes per word
  constexpr int CPC = 4 * CPW;          // codes per 16-byte chunk
  constexpr int BPC = 8 / BITS;         // codes per byte
  constexpr unsigned MASK = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  __shared__ float yloc[4 * RPW];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wpr = L.wpr, ngr = L.ngroups, in = a.in;
  const int nck = (wpr + 4 * 64 - 1) / (4 * 64);      // 16-byte chunks per lane and row
  const int rows = min(4 * RPW, L.out - rw0), wr0 = RPW * wv;   // the workgroup's rows; the wave's

  // 1. loads of the packed words, scales and zeros of the wave's rows, MC chunks at a time.
  //    Descriptors over the workgroup's rows only: rows past `out` read 0.  Words past a
  //    row's end read the next row (or 0); they meet x~ entries past `in`, which are 0.
  const __amdgpu_buffer_rsrc_t rp = rsrc(L.packed + (int64_t)rw0 * wpr, rows * wpr * 4);
  const __amdgpu_buffer_rsrc_t rsc = rsrc(L.scales + (int64_t)rw0 * ngr, rows * ngr * 4);
  const __amdgpu_buffer_rsrc_t rzp = rsrc(L.zeros + (int64_t)rw0 * ngr, rows * ngr);
  u32x4 wq[RPW][MC];
  float sc[RPW][MC], zc[RPW][MC];
  auto load_chunks = [&](int c0) {
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      const int word = ((c0 + c) * 64 + lane) * 4;
      const int pos = word * CPW;
      const int g = (int)__umulhi((unsigned)(pos < in ? pos : in - 1), L.gmagic);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        wq[i][c] = __builtin_amdgcn_raw_buffer_load_b128(rp, ((wr0 + i) * wpr + word) * 4, 0, 0);
        const int go = (wr0 + i) * ngr + g;
        sc[i][c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsc, 4 * go, 0, 0));
        zc[i][c] = (float)__builtin_amdgcn_raw_buffer_load_b8(rzp, go, 0, 0);
      }
    }
  };

  // 2. x~ = Had_b(S_in . x / d_in) / sqrt(b) into LDS (zero past `in`): its loads first, then
  //    the weight loads, whose latency the transform then overlaps
  stage_rotated<B>(xs, a.x, L.d_in, L.s_in, L.isb_in, true, in, a.xlen, L.bin,
                   [&] { load_chunks(0); });

  // 3. dot products: row r's chunk contributes s (sum q x~ - z sum x~)
  float acc[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < nck; c0 += MC) {
    if (c0 > 0) load_chunks(c0);
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      if (c0 + c >= nck) break;   // uniform; only in the last batch
      const int pos = ((c0 + c) * 64 + lane) * CPC;   // first code of the chunk (< xlen)
      float xv[CPC];
#pragma unroll
      for (int k = 0; k < CPC; k += 4) {
        const float4 v = *(const float4*)(xs + pad(pos + k));
        xv[k] = v.x; xv[k + 1] = v.y; xv[k + 2] = v.z; xv[k + 3] = v.w;
      }
      float sx = 0.f;
#pragma unroll
      for (int k = 0; k < CPC; ++k) sx += xv[k];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        float qx = 0.f;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const unsigned u = wq[i][c][wd];
#pragma unroll
          for (int j = 0; j < BPC; ++j) {
            // byte k of m holds code k * BPC + j of the word
            const unsigned m = (u >> (j * BITS)) & MASK;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              qx = fmaf((float)((m >> (8 * k)) & 0xffu), xv[wd * CPW + k * BPC + j], qx);
          }
        }
        acc[i] += sc[i][c] * (qx - zc[i][c] * sx);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[i] += __shfl_xor(acc[i], o);

  if (L.bout > DR) {
    // y~ for the output-rotation kernel
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < RPW; ++i)
        if (wr0 + i < rows) L.y[rw0 + wr0 + i] = acc[i];
    }
    return;
  }
  // 4. this workgroup holds whole output blocks: y = S_out . Had_b(y~) / sqrt(b) / d_out,
  //    Had_b[j][k] = (-1)^popcount(j & k)
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) yloc[wr0 + i] = acc[i];
  }
  __syncthreads();
  if (t < rows) {
    float v = L.isb_out;
    if (L.d_out) v = v / L.d_out[rw0 + t];
    if (L.s_out && L.s_out[rw0 + t] < 0) v = -v;
    const int b = L.bout, j = t % b, blk0 = t - j;
    float s = 0.f;
    for (int k = 0; k < b; ++k) {
      const float yk = yloc[blk0 + k];
      s += (__builtin_popcount(j & k) & 1) ? -yk : yk;
    }
    L.y[rw0 + t] = s * v;
  }
}

// One workgroup per 4 RPW rows of every layer of the call.  W: 4 or 2 when every layer of the
// call has codes of that width, 0 for a mix (both bodies compiled in, more registers).
// RPW = 8 halves the workgroups (and the input transforms) of calls with more row tiles
// than the device holds at once, so they run in one round.
template <int W, int MC, int B, int RPW>
__global__ __launch_bounds__(DT) void deploy_matvec_kernel(GroupArgs a) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  const int l = layer_of(a, blockIdx.x, false);
  const LayerArgs& L = a.L[l];
  const int rw0 = ((int)blockIdx.x - L.wg0) * 4 * RPW;
  if (W == 4 || (W == 0 && L.bits == 4))
    matvec_rows<4, MC, B, RPW>(a, L, rw0, xs);
  else
    matvec_rows<2, MC, B, RPW>(a, L, rw0, xs);
}

// y[s0 .. s0 + n) <- S_out . Had_b(y~) / sqrt(b) / d_out over a segment (whole blocks,
// n <= 2 * 16 * DT) of a layer whose output blocks exceed 16 rows, in place.  The output
// factors are loaded before the transform.
__global__ __launch_bounds__(DT) void deploy_outrot_kernel(GroupArgs a) {
  extern __shared__ __attribute__((aligned(16))) float ys[];
  const LayerArgs& L = a.L[layer_of(a, blockIdx.x, true)];
  const int s0 = ((int)blockIdx.x - L.sg0) * L.seg;
  const int n = min(L.seg, L.out - s0), t = threadIdx.x;
  const float* d = L.d_out ? L.d_out + s0 : nullptr;
  const int8_t* sg = L.s_out ? L.s_out + s0 : nullptr;
  float f[2][16];
  factors16(d, sg, L.isb_out, 16 * t, n, f[0]);
  factors16(d, sg, L.isb_out, 16 * (t + DT), n, f[1]);
  stage_rotated<2>(ys, L.y + s0, nullptr, nullptr, 1.f, false, n, n, L.bout, [] {});
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = 16 * (t + DT * k);
    if (c >= n) break;
    float r[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *(const float4*)(ys + pad(c + 4 * q));
      r[4 * q] = v.x * f[k][4 * q];
      r[4 * q + 1] = v.y * f[k][4 * q + 1];
      r[4 * q + 2] = v.z * f[k][4 * q + 2];
      r[4 * q + 3] = v.w * f[k][4 * q + 3];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(L.y + s0 + c + 4 * q) = make_float4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
  }
}

// Hadamard block of a side: 0 = the largest power of 2 dividing n, as in kq_biip_rotate;
// 1 = none
int64_t deploy_block(int64_t n, int64_t had) { return had != 0 ? had : (n & -n); }

constexpr size_t LDS_MAX = 160 * 1024;

template <typename K>
kq_status launch_with_lds(K kernel, unsigned grid, size_t lds, hipStream_t s, const GroupArgs& a,
                          const char* name) {
  if (lds > 64 * 1024)
    KQ_HIP(hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
  kernel<<<dim3(grid), dim3(DT), lds, s>>>(a);
  KQ_LAUNCHED(name);
  return KQ_OK;
}

kq_status deploy_group(const kq_deploy_layer* layers, int nl, int64_t in, const float* x,
                       void* stream, const char* fn) {
  if (!layers || !x) return fail(KQ_EINVAL, "%s: NULL argument", fn);
  if (nl < 1 || nl > MAXL) return fail(KQ_ESHAPE, "%s: %d layers (1 .. %d per call)", fn, nl, MAXL);
  if (in < 32 || in % 32 != 0 || in > (1 << 20))
    return fail(KQ_ESHAPE, "%s: in = %lld (a multiple of 32)", fn, (long long)in);
  GroupArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.nl = nl;
  a.in = (int)in;
  int64_t chunk = 0, wg = 0, sg = 0, nck = 0, tiles16 = 0;
  int wmask = 0;   // 1: some layer has 4-bit codes; 2: some layer has 2-bit codes
  for (int l = 0; l < nl; ++l) {
    const kq_deploy_layer& q = layers[l];
    LayerArgs& L = a.L[l];
    if (!q.packed || !q.scales || !q.zeros || !q.y) return fail(KQ_EINVAL, "%s: layer %d: NULL argument", fn, l);
    if (q.bits != 2 && q.bits != 4) return fail(KQ_ENOTIMPL, "%s: layer %d: bits must be 2 or 4", fn, l);
    if (q.out < 1 || q.out > (1 << 24)) return fail(KQ_ESHAPE, "%s: layer %d: out = %lld", fn, l, (long long)q.out);
    const int cpc = 4 * 32 / q.bits;
    if (q.group < 1 || in % q.group != 0 || (q.group != in && q.group % cpc != 0))
      return fail(KQ_ESHAPE, "%s: layer %d: group must divide in and be a multiple of %d (or in)", fn, l, cpc);
    if (q.had_in < 0 || q.had_out < 0) return fail(KQ_ESHAPE, "%s: layer %d: negative block", fn, l);
    const int64_t bin = deploy_block(in, q.had_in), bout = deploy_block(q.out, q.had_out);
    if ((q.had_in == 0 && bin > 8192) || (q.had_out == 0 && bout > 8192))
      return fail(KQ_ENOTIMPL, "%s: layer %d: the automatic Hadamard block (the largest power of 2 "
                  "dividing the size) exceeds 8192; pass a block of at most 8192", fn, l);
    if (!is_pow2(bin) || in % bin != 0 || bin > 8192 || !is_pow2(bout) || q.out % bout != 0 || bout > 8192)
      return fail(KQ_ESHAPE, "%s: layer %d: Hadamard blocks must be powers of 2 (<= 8192) dividing the sizes", fn, l);
    L.packed = q.packed; L.scales = q.scales; L.zeros = q.zeros;
    L.d_in = q.d_in; L.d_out = q.d_out; L.s_in = q.sign_in; L.s_out = q.sign_out; L.y = q.y;
    L.out = (int)q.out; L.wpr = (int)(in * q.bits / 32); L.ngroups = (int)(in / q.group); L.bits = q.bits;
    L.bin = (int)bin; L.bout = (int)bout;
    L.isb_in = (float)(1.0 / sqrt((double)bin));
    L.isb_out = (float)(1.0 / sqrt((double)bout));
    // exact for every code position below 2^16 (the LDS limit keeps in below that)
    L.gmagic = (unsigned)(((1ull << 32) + (unsigned)q.group - 1) / (unsigned)q.group);
    tiles16 += ceil_div(q.out, 16);
    L.seg = (int)std::max<int64_t>(bout, SEG);
    L.sg0 = (int)sg;
    if (bout > DR) sg += ceil_div(q.out, L.seg);
    chunk = std::max<int64_t>(chunk, 64 * cpc);   // codes per chunk column of a wave
    wmask |= q.bits == 4 ? 1 : 2;
    nck = std::max<int64_t>(nck, (L.wpr + 255) / 256);
  }
  const int64_t xlen = (in + chunk - 1) / chunk * chunk;
  const bool b1 = xlen / 16 <= DT;   // one staging group per thread
  const size_t lds = (size_t)padded_len((int)std::max<int64_t>(xlen, 16 * DT * (b1 ? 1 : 2))) * sizeof(float);
  if (lds > LDS_MAX)
    return fail(KQ_ESHAPE, "%s: in = %lld too large for the LDS copy of x", fn, (long long)in);
  a.xlen = (int)xlen;
  hipStream_t s = as_stream(stream);
  // 16-byte chunks per lane and row in flight: all of them up to four, else batches of four
  // (six in flight for the 11008-wide W4 rows took 289 registers, one wave per SIMD; batches
  // of four leave room for two and ran that call 3 % faster)
  const int mc = nck <= 2 ? 2 : 4;
  // 8 rows per wave when the 16-row tiles outnumber what the device holds at once (about
  // four workgroups per CU) and the weights of 8 rows fit in registers
  const int rpw = (tiles16 > 4 * (int64_t)device_cu_count() && mc <= 4) ? 8 : 4;
  for (int l = 0; l < nl; ++l) {
    a.L[l].wg0 = (int)wg;
    wg += ceil_div(a.L[l].out, 4 * rpw);
  }
  const char* nm = "deploy_matvec_kernel";
  const unsigned grid = (unsigned)wg;
  kq_status st;
#define KQ_MV4(W, M)                                                                         \
  (b1 ? launch_with_lds(deploy_matvec_kernel<W, M, 1, 4>, grid, lds, s, a, nm)               \
      : launch_with_lds(deploy_matvec_kernel<W, M, 2, 4>, grid, lds, s, a, nm))
#define KQ_MV8(W, M)                                                                         \
  (b1 ? launch_with_lds(deploy_matvec_kernel<W, M, 1, 8>, grid, lds, s, a, nm)               \
      : launch_with_lds(deploy_matvec_kernel<W, M, 2, 8>, grid, lds, s, a, nm))
#define KQ_MV(W)                                                                             \
  (rpw == 8 ? (mc == 2 ? KQ_MV8(W, 2) : KQ_MV8(W, 4))                                        \
            : (mc == 2 ? KQ_MV4(W, 2) : KQ_MV4(W, 4)))
  st = wmask == 1 ? KQ_MV(4) : wmask == 2 ? KQ_MV(2) : KQ_MV(0);
#undef KQ_MV
#undef KQ_MV8
#undef KQ_MV4
  if (st != KQ_OK || sg == 0) return st;
  const size_t lds2 = (size_t)padded_len(2 * 16 * DT) * sizeof(float);   // seg <= 8192
  return launch_with_lds(deploy_outrot_kernel, (unsigned)sg, lds2, s, a, "deploy_outrot_kernel");
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_deploy_linear_group(const kq_deploy_layer* layers, int n_layers,
                                            int64_t in, const float* x, void* stream) {
  return kq::deploy_group(layers, n_layers, in, x, stream, "kq_deploy_linear_group");
}

extern "C" kq_status kq_deploy_linear(const uint32_t* packed, const float* scales,
                                      const uint8_t* zeros, int bits, int group, int64_t out,
                                      int64_t in, const float* d_in, const float* d_out,
                                      const int8_t* sign_in, const int8_t* sign_out,
                                      int64_t had_in, int64_t had_out, const float* x, float* y,
                                      void* stream) {
  kq_deploy_layer l;
  l.packed = packed; l.scales = scales; l.zeros = zeros; l.bits = bits; l.group = group;
  l.out = out; l.d_in = d_in; l.d_out = d_out; l.sign_in = sign_in; l.sign_out = sign_out;
  l.had_in = had_in; l.had_out = had_out; l.y = y;
  return kq::deploy_group(&l, 1, in, x, stream, "kq_deploy_linear");
}
