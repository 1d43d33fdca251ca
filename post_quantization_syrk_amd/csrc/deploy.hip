// Deploy side: one BiIP-quantized layer applied to an activation vector (batch 1),
//   y = D_out^-1 P_out^T Qhat P_in D_in^-1 x,   Qhat[r, c] = s[r, g] (q[r, c] - z[r, g]).
//
// KronQ README, opening section: the packed int4/int2 weights are dequantized on the fly by a
// fused dequant + BiIP matvec for single-token decode.  Here, one kernel per layer:
//   * each workgroup owns 16 rows (4 per wave) and first issues the loads of its rows' packed
//     words (16 bytes per lane, a row's words contiguous across the wave's lanes);
//   * while they are in flight it forms x~ = Had_b(S_in . x / d_in) / sqrt(b) in LDS
//     (every workgroup for itself: a few microseconds of ALU work hidden by the loads);
//   * a lane's codes are unpacked byte-wise (v_cvt_f32_ubyte) and a row's dot product is taken
//     as s (sum q x~ - z sum x~) per chunk, the x~ values read once for the wave's 4 rows;
//   * the output rotation needs every row of an output Hadamard block: blocks of at most 16
//     rows are finished by the workgroup that owns them; larger ones by the workgroup whose
//     rows complete the block (a per-block row counter, reset by that workgroup).
// The layer is HBM-bound: out * in * bits / 8 bytes of packed words per call.
#include "kq_internal.h"

#include <math.h>

namespace kq {
namespace {

constexpr int DT = 256;   // threads per workgroup
constexpr int DR = 16;    // rows per workgroup (4 per wave)
constexpr int MAXC = 8;   // 16-byte chunks per lane and row kept in flight

struct DeployArgs {
  const uint32_t* packed;  // out x wpr words
  const float* scales;     // out x ngroups
  const uint8_t* zeros;    // out x ngroups
  int64_t out, in, wpr, ngroups;
  int group;
  const float* d_in;
  const float* d_out;
  const int8_t* s_in;
  const int8_t* s_out;
  int bin, bout;
  float isb_in, isb_out;   // 1 / sqrt(block)
  const float* x;
  float* y;
  float* yt;               // out floats: the rotated output before the output rotation
  int* cnt;                // per output block: rows finished
  int64_t xlen;            // LDS length of x~ (in rounded up to whole chunks)
};

constexpr int OOB = 0x7ffffff0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  // 0x00020000: the descriptor's data-format word on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, OOB, 0x00020000);
}

// In-place Walsh-Hadamard transform (Sylvester order, unnormalized) of every b-block of
// v[0..n) in LDS, all threads; n a multiple of b, b a power of 2.
__device__ __forceinline__ void lds_fwht(float* v, int64_t n, int b) {
  const int t = threadIdx.x;
  for (int h = 1; h < b; h <<= 1) {
    const int lh = __builtin_ctz(h);
    for (int64_t p = t; p < n / 2; p += DT) {
      const int64_t i = ((p >> lh) << (lh + 1)) | (p & (h - 1));
      const float a = v[i], c = v[i + h];
      v[i] = a + c;
      v[i + h] = a - c;
    }
    __syncthreads();
  }
}

// o[k] = v[c0 + c] for c = threadIdx.x + DT k, k < NF (0 at or past n): global memory only,
// loads without branches (masked through out-of-range offsets).
template <int NF>
__device__ __forceinline__ void masked_loads(const float* v, int64_t n, int64_t c0, float (&o)[NF]) {
  const __amdgpu_buffer_rsrc_t rv = rsrc(v + c0);
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    const int c = threadIdx.x + DT * k;
    o[k] = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rv, c0 + c < n ? 4 * c : OOB, 0, 0));
  }
}

// f[k] = mul * sign[c0 + c] / d[c0 + c] for c = threadIdx.x + DT k (an absent vector counts as
// 1; 0 at or past n, where the unmasked division would give inf): global memory, loads
// without branches.
template <int NF>
__device__ __forceinline__ void scale_factors(const float* d, const int8_t* sg, float mul,
                                              int64_t n, int64_t c0, float (&f)[NF]) {
  const bool hd = d != nullptr, hs = sg != nullptr;
  const __amdgpu_buffer_rsrc_t rd = rsrc(hd ? d + c0 : d), rg = rsrc(hs ? sg + c0 : sg);
  float dv[NF];
  int gv[NF];
  bool ok[NF];
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    const int c = threadIdx.x + DT * k;
    ok[k] = c0 + c < n;
    dv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, ok[k] && hd ? 4 * c : OOB, 0, 0));
    gv[k] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(rg, ok[k] && hs ? c : OOB, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    float x = mul;
    if (hd) x = x / (ok[k] ? dv[k] : 1.0f);
    x = gv[k] < 0 ? -x : x;
    f[k] = ok[k] ? x : 0.0f;
  }
}

template <int BITS, int MC>
__global__ __launch_bounds__(DT) void deploy_kernel(DeployArgs a) {
  constexpr int CPW = 32 / BITS;        // codes per word
  constexpr int CPC = 4 * CPW;          // codes per 16-byte chunk
  constexpr int BPC = 8 / BITS;         // codes per byte
  constexpr unsigned MASK = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float yloc[DR];
  __shared__ int s_last;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t rw0 = (int64_t)blockIdx.x * DR;          // the workgroup's first row
  const int64_t r0 = rw0 + 4 * wv;                        // this wave's first row
  const int64_t nck = (a.wpr + 4 * 64 - 1) / (4 * 64);    // 16-byte chunks per lane and row

  // 1. packed words, scales and zeros of the wave's 4 rows, MC chunks at a time (rows past
  //    `out` and words past the row read 0 through out-of-range offsets)
  const __amdgpu_buffer_rsrc_t rp = rsrc(a.packed + rw0 * a.wpr);
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 wq[4][MC];
  float sc[4][MC], zc[4][MC];
  auto load_chunks = [&](int64_t c0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < MC; ++c) {
        const int64_t word = ((c0 + c) * 64 + lane) * 4;
        const bool ok = r0 + i < a.out && word < a.wpr;
        wq[i][c] = __builtin_amdgcn_raw_buffer_load_b128(
            rp, ok ? (int)(((r0 + i - rw0) * a.wpr + word) * 4) : OOB, 0, 0);
        const int64_t r = r0 + i < a.out ? r0 + i : a.out - 1;
        const int64_t pos = word * CPW;
        const int64_t g = (pos < a.in ? pos : a.in - 1) / a.group;
        sc[i][c] = a.scales[r * a.ngroups + g];
        zc[i][c] = (float)a.zeros[r * a.ngroups + g];
      }
  };
  load_chunks(0);

  // 2. x~ = S_in . x / d_in / sqrt(b) into LDS (zero past `in`), then the block Hadamard,
  //    while the weight loads are in flight
  for (int64_t c0 = 0; c0 < a.xlen; c0 += 8 * DT) {
    float v[8], f[8];
    masked_loads<8>(a.x, a.in, c0, v);
    scale_factors<8>(a.d_in, a.s_in, a.isb_in, a.in, c0, f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t c = c0 + t + DT * k;
      if (c < a.xlen) xs[c] = v[k] * f[k];
    }
  }
  __syncthreads();
  if (a.bin > 1) lds_fwht(xs, a.in, a.bin);

  // 3. dot products: row r's chunk contributes s (sum q x~ - z sum x~)
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c0 = 0; c0 < nck; c0 += MC) {
    if (c0 > 0) load_chunks(c0);
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      if (c0 + c >= nck) break;   // uniform; only in the last batch
      const int64_t pos = ((c0 + c) * 64 + lane) * CPC;   // first code of the chunk (< xlen)
      float xv[CPC];
#pragma unroll
      for (int k = 0; k < CPC; k += 4) {
        const float4 v = *(const float4*)(xs + pos + k);
        xv[k] = v.x; xv[k + 1] = v.y; xv[k + 2] = v.z; xv[k + 3] = v.w;
      }
      float sx = 0.f;
#pragma unroll
      for (int k = 0; k < CPC; ++k) sx += xv[k];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
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
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[i] += __shfl_xor(acc[i], o);

  // 4. output rotation and rescale: y = S_out . Had_b(y~) / sqrt(b) / d_out
  const int64_t nrows = min((int64_t)DR, a.out - rw0);
  if (a.bout <= DR) {
    // this workgroup holds whole output blocks: Had_b[j][k] = (-1)^popcount(j & k)
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) yloc[4 * wv + i] = acc[i];
    }
    __syncthreads();
    float f[1];
    scale_factors<1>(a.d_out, a.s_out, a.isb_out, a.out, rw0, f);
    if (t < nrows) {
      const int b = a.bout, j = t % b, blk0 = t - j;
      float v = 0.f;
      for (int k = 0; k < b; ++k) {
        const float yk = yloc[blk0 + k];
        v += (__builtin_popcount(j & k) & 1) ? -yk : yk;
      }
      a.y[rw0 + t] = v * f[0];
    }
    return;
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (r0 + i < a.out) a.yt[r0 + i] = acc[i];
  }
  __threadfence();
  __syncthreads();
  const int64_t blk = rw0 / a.bout;
  if (t == 0) {
    const int old = atomicAdd(a.cnt + blk, (int)nrows);
    s_last = old + (int)nrows == a.bout ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  // the last workgroup of the block: every row's y~ is visible after this fence
  __threadfence();
  const int64_t base = blk * a.bout;
  for (int64_t c0 = 0; c0 < a.bout; c0 += 8 * DT) {
    float v[8];
    masked_loads<8>(a.yt + base, a.bout, c0, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t c = c0 + t + DT * k;
      if (c < a.bout) xs[c] = v[k];
    }
  }
  __syncthreads();
  lds_fwht(xs, a.bout, a.bout);
  for (int64_t c0 = 0; c0 < a.bout; c0 += 8 * DT) {
    float f[8];
    scale_factors<8>(a.d_out ? a.d_out + base : nullptr, a.s_out ? a.s_out + base : nullptr,
                     a.isb_out, a.bout, c0, f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t c = c0 + t + DT * k;
      if (c < a.bout) a.y[base + c] = xs[c] * f[k];
    }
  }
  if (t == 0) atomicExch(a.cnt + blk, 0);
}

}  // namespace
}  // namespace kq

namespace kq {
namespace {
// Hadamard block of a side: 0 = the largest power of 2 dividing n (at most 8192), as in
// kq_biip_rotate; 1 = none
int64_t deploy_block(int64_t n, int64_t had) {
  if (had != 0) return had;
  int64_t b = n & -n;
  while (b > 8192) b >>= 1;
  return b;
}
}  // namespace
}  // namespace kq

extern "C" kq_status kq_deploy_linear_workspace(int64_t out, int64_t had_out, size_t* bytes) {
  using namespace kq;
  if (!bytes) return fail(KQ_EINVAL, "kq_deploy_linear_workspace: bytes is NULL");
  if (out < 1 || had_out < 0) return fail(KQ_ESHAPE, "kq_deploy_linear_workspace: bad sizes");
  const int64_t b = deploy_block(out, had_out);
  const int64_t nblk = (out + b - 1) / b;
  *bytes = ((size_t)nblk * sizeof(int) + 255) / 256 * 256 + (size_t)out * sizeof(float);
  return KQ_OK;
}

extern "C" kq_status kq_deploy_linear(const uint32_t* packed, const float* scales,
                                      const uint8_t* zeros, int bits, int group, int64_t out,
                                      int64_t in, const float* d_in, const float* d_out,
                                      const int8_t* sign_in, const int8_t* sign_out,
                                      int64_t had_in, int64_t had_out, const float* x, float* y,
                                      void* ws, size_t ws_bytes, void* stream) {
  using namespace kq;
  if (!packed || !scales || !zeros || !x || !y) return fail(KQ_EINVAL, "kq_deploy_linear: NULL argument");
  if (bits != 2 && bits != 4) return fail(KQ_ENOTIMPL, "kq_deploy_linear: bits must be 2 or 4");
  if (out < 1 || in < 1 || in % 32 != 0 || out > (1 << 24) || in > (1 << 20))
    return fail(KQ_ESHAPE, "kq_deploy_linear: bad shape %lld x %lld", (long long)out, (long long)in);
  const int cpc = 4 * 32 / bits;
  if (group < 1 || in % group != 0 || (group != in && group % cpc != 0))
    return fail(KQ_ESHAPE, "kq_deploy_linear: group must divide in and be a multiple of %d (or in)", cpc);
  if (had_in < 0 || had_out < 0) return fail(KQ_ESHAPE, "kq_deploy_linear: negative block");
  const int64_t bin = deploy_block(in, had_in), bout = deploy_block(out, had_out);
  if (!is_pow2(bin) || in % bin != 0 || bin > 8192 || !is_pow2(bout) || out % bout != 0 || bout > 8192)
    return fail(KQ_ESHAPE, "kq_deploy_linear: Hadamard blocks must be powers of 2 dividing the sizes");
  size_t need = 0;
  KQ_TRY(kq_deploy_linear_workspace(out, bout, &need));
  if (bout > DR && (!ws || ws_bytes < need))
    return fail(KQ_EWORKSPACE, "kq_deploy_linear: workspace of %zu bytes needed", need);
  DeployArgs a;
  a.packed = packed; a.scales = scales; a.zeros = zeros;
  a.out = out; a.in = in; a.wpr = in * bits / 32; a.ngroups = in / group; a.group = group;
  a.d_in = d_in; a.d_out = d_out; a.s_in = sign_in; a.s_out = sign_out;
  a.bin = (int)bin; a.bout = (int)bout;
  a.isb_in = (float)(1.0 / sqrt((double)bin));
  a.isb_out = (float)(1.0 / sqrt((double)bout));
  a.x = x; a.y = y;
  const int64_t nblk = (out + bout - 1) / bout;
  a.cnt = (int*)ws;
  a.yt = ws ? (float*)((char*)ws + (nblk * sizeof(int) + 255) / 256 * 256) : nullptr;
  const int64_t chunk = 64 * cpc;   // codes per chunk column of a wave
  a.xlen = (in + chunk - 1) / chunk * chunk;
  const size_t lds = (size_t)(a.xlen > bout ? a.xlen : bout) * sizeof(float);
  if (lds > 160 * 1024) return fail(KQ_ESHAPE, "kq_deploy_linear: in too large for LDS");
  hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)ceil_div(out, DR));
  // 16-byte chunks per lane and row: all of them in flight when they fit in MAXC
  const int64_t nck = (a.wpr + 255) / 256;
  const int mc = nck <= 2 ? 2 : nck <= 4 ? 4 : MAXC;
#define KQ_DEPLOY(B, M) deploy_kernel<B, M><<<grid, dim3(DT), lds, s>>>(a)
  if (bits == 4) {
    if (mc == 2) KQ_DEPLOY(4, 2); else if (mc == 4) KQ_DEPLOY(4, 4); else KQ_DEPLOY(4, MAXC);
  } else {
    if (mc == 2) KQ_DEPLOY(2, 2); else if (mc == 4) KQ_DEPLOY(2, 4); else KQ_DEPLOY(2, MAXC);
  }
#undef KQ_DEPLOY
  KQ_LAUNCHED("deploy_kernel");
  return KQ_OK;
}
