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
#include "kq_internal.h"

#include <math.h>

#include <algorithm>

namespace kq {
namespace {

constexpr int DT = 256;     // threads per workgroup
constexpr int DR = 16;      // rows per workgroup of the matvec kernel (4 per wave)
constexpr int MAXC = 8;     // 16-byte chunks per lane and row kept in flight
constexpr int SEG = 4096;   // entries per workgroup of the output rotation (or one block)

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
  int xlen;                // entries of x~ in LDS (in rounded up to whole chunks)
  int seg;                 // entries per workgroup of the output rotation
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int OOB = 0x7ffffff0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  // 0x00020000: the descriptor's data-format word on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, OOB, 0x00020000);
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

// f[j] = mul * sign[c + j] / d[c + j] for j < 16 (an absent vector counts as 1); loads only
// when `ok`.  d and sg are uniform across the workgroup.
__device__ __forceinline__ void factors16(const float* d, const int8_t* sg, float mul, int c,
                                          bool ok, float (&f)[16]) {
  const bool hd = d != nullptr, hs = sg != nullptr;
  const __amdgpu_buffer_rsrc_t rd = rsrc(d), rg = rsrc(sg);
  u32x4 dv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dv[q] = __builtin_amdgcn_raw_buffer_load_b128(rd, ok && hd ? 4 * (c + 4 * q) : OOB, 0, 0);
  const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rg, ok && hs ? c : OOB, 0, 0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float v = mul;
    if (hd) v = v / __uint_as_float(dv[j >> 2][j & 3]);
    const int sgn = (int)(int8_t)((sv[j >> 2] >> (8 * (j & 3))) & 0xffu);
    if (hs && sgn < 0) v = -v;
    f[j] = v;
  }
}

// v (LDS, padded) <- the b-block transform of src[0..n) (times the input factors when `pre`),
// entries n .. len zero.  n and len are multiples of 16; src is uniform across the workgroup.
__device__ __forceinline__ void stage_rotated(float* v, const float* src, const float* d,
                                              const int8_t* sg, float mul, bool pre, int n,
                                              int len, int b) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(src);
  const int R = b >= 16 ? 16 : b;
  for (int g = threadIdx.x; g < len / 16; g += DT) {
    const int c = 16 * g;
    const bool ok = c < n;
    u32x4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xv[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? 4 * (c + 4 * q) : OOB, 0, 0);
    float r[16];
    if (pre) {
      float f[16];
      factors16(d, sg, mul, c, ok, f);
#pragma unroll
      for (int j = 0; j < 16; ++j) r[j] = ok ? __uint_as_float(xv[j >> 2][j & 3]) * f[j] : 0.f;
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) r[j] = __uint_as_float(xv[j >> 2][j & 3]);
    }
    bfly_runs16(r, R);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(v + pad(c + 4 * q)) = make_float4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
  }
  __syncthreads();
  lds_fwht_rest(v, n, b);
}

template <int BITS, int MC>
__global__ __launch_bounds__(DT) void deploy_matvec_kernel(DeployArgs a) {
  constexpr int CPW = 32 / BITS;        // codes per word
  constexpr int CPC = 4 * CPW;          // codes per 16-byte chunk
  constexpr int BPC = 8 / BITS;         // codes per byte
  constexpr unsigned MASK = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float yloc[DR];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t rw0 = (int64_t)blockIdx.x * DR;          // the workgroup's first row
  const int64_t r0 = rw0 + 4 * wv;                        // this wave's first row
  const int64_t nck = (a.wpr + 4 * 64 - 1) / (4 * 64);    // 16-byte chunks per lane and row

  // 1. packed words, scales and zeros of the wave's 4 rows, MC chunks at a time (rows past
  //    `out` and words past the row read 0 through out-of-range offsets)
  const __amdgpu_buffer_rsrc_t rp = rsrc(a.packed + rw0 * a.wpr);
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

  // 2. x~ = Had_b(S_in . x / d_in) / sqrt(b) into LDS (zero past `in`) while the weight loads
  //    are in flight
  stage_rotated(xs, a.x, a.d_in, a.s_in, a.isb_in, true, (int)a.in, a.xlen, a.bin);

  // 3. dot products: row r's chunk contributes s (sum q x~ - z sum x~)
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c0 = 0; c0 < nck; c0 += MC) {
    if (c0 > 0) load_chunks(c0);
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      if (c0 + c >= nck) break;   // uniform; only in the last batch
      const int pos = (int)(((c0 + c) * 64 + lane) * CPC);   // first code of the chunk (< xlen)
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

  if (a.bout > DR) {
    // y~ for the output-rotation kernel
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (r0 + i < a.out) a.y[r0 + i] = acc[i];
    }
    return;
  }
  // 4. this workgroup holds whole output blocks: y = S_out . Had_b(y~) / sqrt(b) / d_out,
  //    Had_b[j][k] = (-1)^popcount(j & k)
  const int64_t nrows = min((int64_t)DR, a.out - rw0);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) yloc[4 * wv + i] = acc[i];
  }
  __syncthreads();
  if (t < nrows) {
    float v = a.isb_out;
    if (a.d_out) v = v / a.d_out[rw0 + t];
    if (a.s_out && a.s_out[rw0 + t] < 0) v = -v;
    const int b = a.bout, j = t % b, blk0 = t - j;
    float s = 0.f;
    for (int k = 0; k < b; ++k) {
      const float yk = yloc[blk0 + k];
      s += (__builtin_popcount(j & k) & 1) ? -yk : yk;
    }
    a.y[rw0 + t] = s * v;
  }
}

// y[s0 .. s0 + n) <- S_out . Had_b(y~) / sqrt(b) / d_out over the workgroup's segment (whole
// blocks), in place.
__global__ __launch_bounds__(DT) void deploy_outrot_kernel(DeployArgs a) {
  extern __shared__ __attribute__((aligned(16))) float ys[];
  const int64_t s0 = (int64_t)blockIdx.x * a.seg;
  const int n = (int)min((int64_t)a.seg, a.out - s0);
  stage_rotated(ys, a.y + s0, nullptr, nullptr, 1.f, false, n, n, a.bout);
  for (int g = threadIdx.x; g < n / 16; g += DT) {
    const int c = 16 * g;
    float f[16];
    factors16(a.d_out ? a.d_out + s0 : nullptr, a.s_out ? a.s_out + s0 : nullptr, a.isb_out, c,
              true, f);
    float r[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *(const float4*)(ys + pad(c + 4 * q));
      r[4 * q] = v.x * f[4 * q];
      r[4 * q + 1] = v.y * f[4 * q + 1];
      r[4 * q + 2] = v.z * f[4 * q + 2];
      r[4 * q + 3] = v.w * f[4 * q + 3];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(a.y + s0 + c + 4 * q) = make_float4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
  }
}

// Hadamard block of a side: 0 = the largest power of 2 dividing n (at most 8192), as in
// kq_biip_rotate; 1 = none
int64_t deploy_block(int64_t n, int64_t had) {
  if (had != 0) return had;
  int64_t b = n & -n;
  while (b > 8192) b >>= 1;
  return b;
}

constexpr size_t LDS_MAX = 160 * 1024;

template <typename K>
kq_status launch_with_lds(K kernel, dim3 grid, size_t lds, hipStream_t s, const DeployArgs& a,
                          const char* name) {
  if (lds > 64 * 1024)
    KQ_HIP(hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
  kernel<<<grid, dim3(DT), lds, s>>>(a);
  KQ_LAUNCHED(name);
  return KQ_OK;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_deploy_linear(const uint32_t* packed, const float* scales,
                                      const uint8_t* zeros, int bits, int group, int64_t out,
                                      int64_t in, const float* d_in, const float* d_out,
                                      const int8_t* sign_in, const int8_t* sign_out,
                                      int64_t had_in, int64_t had_out, const float* x, float* y,
                                      void* stream) {
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
  const int64_t chunk = 64 * cpc;   // codes per chunk column of a wave
  const int64_t xlen = (in + chunk - 1) / chunk * chunk;
  const size_t lds = (size_t)padded_len((int)xlen) * sizeof(float);
  if (lds > LDS_MAX)
    return fail(KQ_ESHAPE, "kq_deploy_linear: in = %lld too large for the LDS copy of x", (long long)in);
  DeployArgs a;
  a.packed = packed; a.scales = scales; a.zeros = zeros;
  a.out = out; a.in = in; a.wpr = in * bits / 32; a.ngroups = in / group; a.group = group;
  a.d_in = d_in; a.d_out = d_out; a.s_in = sign_in; a.s_out = sign_out;
  a.bin = (int)bin; a.bout = (int)bout;
  a.isb_in = (float)(1.0 / sqrt((double)bin));
  a.isb_out = (float)(1.0 / sqrt((double)bout));
  a.x = x; a.y = y;
  a.xlen = (int)xlen;
  a.seg = (int)std::max<int64_t>(bout, SEG);
  hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)ceil_div(out, DR));
  // 16-byte chunks per lane and row: all of them in flight when they fit in MAXC
  const int64_t nck = (a.wpr + 255) / 256;
  const int mc = nck <= 2 ? 2 : nck <= 4 ? 4 : MAXC;
  const char* nm = "deploy_matvec_kernel";
  kq_status st;
  if (bits == 4)
    st = mc == 2 ? launch_with_lds(deploy_matvec_kernel<4, 2>, grid, lds, s, a, nm)
       : mc == 4 ? launch_with_lds(deploy_matvec_kernel<4, 4>, grid, lds, s, a, nm)
                 : launch_with_lds(deploy_matvec_kernel<4, MAXC>, grid, lds, s, a, nm);
  else
    st = mc == 2 ? launch_with_lds(deploy_matvec_kernel<2, 2>, grid, lds, s, a, nm)
       : mc == 4 ? launch_with_lds(deploy_matvec_kernel<2, 4>, grid, lds, s, a, nm)
                 : launch_with_lds(deploy_matvec_kernel<2, MAXC>, grid, lds, s, a, nm);
  if (st != KQ_OK || bout <= DR) return st;
  const size_t lds2 = (size_t)padded_len(a.seg) * sizeof(float);
  return launch_with_lds(deploy_outrot_kernel, dim3((unsigned)ceil_div(out, a.seg)), lds2, s, a,
                         "deploy_outrot_kernel");
}
