// GPTQ error-feedback quantization of a processed layer to packed codes.
//
// KronQ README, opening section: KronQ extends GPTQ/GPTAQ, quantizing weights
// only (W2-W4) under the Kronecker objective tr(H_G dW H_X dW^T), with packed
// int2/int4 storage; "Mapping paper results to flags": GPTQ is the base
// quantizer, --w_asym / --w_groupsize set the grid.
//
// GPTQ's column recursion with U = chol_upper(H_d^-1):
//   e_j = (w_j - qhat_j) / U_jj,   w_k -= e_j U_jk  (k > j)
// where the (row, group) grid is taken from the current weights when a group's
// first column is reached.  It is run blockwise, B columns at a time:
//   Y = D[:, <J] P[<J, J]               one fp32 MFMA product, split over K into up to 8
//                                       partial slices that the column kernel sums:
//                                       D = W0 - Qhat (the rounding error so far) and
//                                       P = R[<J, J] U_JJ, so that Y = -E[:, <J] U[<J, J]
//                                       and the block's current weights are W0[:, J] + Y,
//                                       exactly GPTQ's state when the block starts
//   column kernel, column by column inside the block:
//     (at group starts) min-max grid from the current weights of the group,
//     q = clamp(rint(w/s) + z), e_j = (w_j - s (q - z)) / U_jj, w_k -= e_j U_jk (k in J)
//   the codes are packed into the output words in the same kernel; e_j replaces W0_j and
//   W0_j - s (q - z) goes to D.
#include "device_util.h"
#include "kq_internal.h"

#include <mutex>

#include <math.h>

#include <utility>

namespace kq {

kq_status damp_and_factor(const float* HX, float* F, float* T, uint8_t* dead, double* lam,
                          int* flag, int64_t n, float damp, int B, hipStream_t s);

namespace {

constexpr int LPR = 16;             // lanes per matrix row in the column kernel
constexpr int CTHREADS = 256;       // threads per workgroup in the column kernel
constexpr int RPW = CTHREADS / LPR; // matrix rows per workgroup
constexpr int YSLOTS = 8;           // most K splits of the feedback product

// K splits of one feedback product (out x N, K = 32 * stages), at most cap: the count with
// the least modelled time.  Workgroups run in whole rounds of one 128 x 128 tile per CU; a
// split's tile costs its stages plus about three stages of fill and epilogue; every slice
// after the first adds its store here and its read in the column kernel, 8 out N bytes, at
// about 12.8 MB per stage time.
inline int64_t feedback_splits(int64_t out, int64_t N, int64_t stages, int64_t cap, int cus) {
  const int64_t tiles = ceil_div(out, 128) * ceil_div(N, 128);
  const double slice = 8.0 * (double)out * (double)N / 12.8e6;
  int64_t best = 1;
  double best_t = -1.0;
  for (int64_t s = 1; s <= cap && s <= stages; ++s) {
    const double t = (double)(ceil_div(tiles * s, cus) * (ceil_div(stages, s) + 3)) + (s - 1) * slice;
    if (best_t < 0.0 || t < best_t) {
      best_t = t;
      best = s;
    }
  }
  return best;
}

// Slices of the feedback product's workspace, for a pair of B-column blocks: the split count
// the model above takes at K = 8192 on a 256-CU device (larger K runs with that many).
inline int64_t y_slots(int64_t out, int B) { return feedback_splits(out, 2 * B, 256, YSLOTS, 256); }

struct ColArgs {
  float* W;            // out x in: W0 (unprocessed columns) / errors e (processed columns)
  int64_t out, in;
  float* Y;            // nsplit slices of out x (nblk B): partial corrections of the launch's
                       // blocks from the columns before them, summed in slice order (D P = -E U)
  int nsplit;          // slices written for this launch (0: no correction)
  int64_t ystride;     // floats between slices
  int nblk;            // blocks of B columns per launch (1 or 2); row pitch of Y is nblk B
  float* D;            // out x in: W0 - Qhat of the processed columns
  const float* U;      // in x in: U_JJ in the diagonal B x B blocks
  const uint8_t* dead; // in
  int bits;
  float maxq;
  int64_t ngroups;     // in / group
  float* scales;       // out x ngroups
  uint8_t* zeros;      // out x ngroups
  uint32_t* packed;    // out x (in * bits / 32), or NULL (codes packed afterwards)
  uint8_t* codes;      // out x in or NULL
};

// Broadcast lane O of every 16-lane row to the whole row (DPP row_newbcast).
template <int O>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + O, 0xF, 0xF, false));
}

// min / max over the 16 lanes of a row
__device__ __forceinline__ float row_min(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v = fminf(v, __shfl_xor(v, m, LPR));
  return v;
}
__device__ __forceinline__ float row_max(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, LPR));
  return v;
}

template <int CPL>
struct RowState {
  float w[CPL];    // current weights of this lane's columns
  float w0[CPL];   // their starting weights (W0)
  float el[CPL];   // errors e_j once quantized
  float dl[CPL];   // W0_j - qhat_j once quantized
  float ql[CPL];   // codes once quantized
  float corr[CPL]; // next block's feedback from this block's W0 - qhat, as it forms
  float s, inv, z; // grid of the current group
};

struct StepCtx {
  const float* Cb;  // LDS: B x B in-block U (zero on and below the diagonal)
  const float* Pb;  // LDS: B x B feedback factor into the next block (CORR steps only)
  int q;            // lane within the row
  bool live;
  int64_t r, j0;
  const ColArgs* a;
};

// Operands a column step reads ahead of time: this lane's slice of U row J and, on lane
// J % 16 of every row, 1 / U_jj for columns J = lane + 16 i (broadcast with DPP).
template <int CPL>
struct Ahead {
  float4 u[3][CPL / 4];   // U rows J, J+1, J+2 (ring indexed by J % 3)
  float ri[CPL];          // ri[i] = 1 / U_jj of column 16 i + lane
};

// One column j of the block (all compile-time indices, so every array stays in registers).
// CORR: also accumulate the next block's feedback, corr += (W0_j - qhat_j) P[j, next block].
template <int B, int G, bool CORR, int J>
__device__ __forceinline__ void gptq_step(RowState<B / LPR>& st, Ahead<B / LPR>& ah,
                                          const StepCtx& cx) {
  constexpr int CPL = B / LPR;
  constexpr int O = J / CPL, E = J % CPL;
  // read U row J + 2 now; it is used two columns later
  if constexpr (J + 2 < B) {
    const float* crow = cx.Cb + (J + 2) * B + 4 * cx.q;
#pragma unroll
    for (int e = 0; e < CPL; e += 4) ah.u[(J + 2) % 3][e / 4] = *(const float4*)(crow + LPR * e);
  }
  float4 pj[CORR ? CPL / 4 : 1];
  if constexpr (CORR) {
    const float* prow = cx.Pb + J * B + 4 * cx.q;
#pragma unroll
    for (int e = 0; e < CPL; e += 4) pj[e / 4] = *(const float4*)(prow + LPR * e);
  }
  // keep those reads here (ALU work and LDS writes may still move across)
  __builtin_amdgcn_sched_barrier(0x607);
  if constexpr (G > 0) {
    if constexpr (J % G == 0) {
      // group [J, J+G) lives on lanes [J/CPL, (J+G)/CPL); the range always includes 0
      const bool in = cx.q >= J / CPL && cx.q < (J + G) / CPL;
      float mn = 0.0f, mx = 0.0f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        mn = fminf(mn, in ? st.w[e] : 0.0f);
        mx = fmaxf(mx, in ? st.w[e] : 0.0f);
      }
      mn = row_min(mn);
      mx = row_max(mx);
      float s = (mx - mn) / cx.a->maxq;
      if (mx == mn) s = 1.0f;
      st.s = s;
      st.inv = 1.0f / s;
      st.z = rintf(-mn / s);
      if (cx.live && cx.q == 0) {
        const int64_t gi = cx.r * cx.a->ngroups + (cx.j0 + J) / G;
        cx.a->scales[gi] = s;
        cx.a->zeros[gi] = (uint8_t)st.z;
      }
    }
  }
  const float wj = row_bcast<O>(st.w[E]);
  const float rij = row_bcast<J % LPR>(ah.ri[J / LPR]);
  float qv = rintf(wj * st.inv) + st.z;
  qv = fminf(fmaxf(qv, 0.0f), cx.a->maxq);
  const float qh = st.s * (qv - st.z);
  const float err = (wj - qh) * rij;
  const float d = -err;
  // every lane of the row holds the same qv and err; the owning lane keeps them
  st.el[E] = cx.q == O ? err : st.el[E];
  st.dl[E] = cx.q == O ? st.w0[E] - qh : st.dl[E];
  st.ql[E] = cx.q == O ? qv : st.ql[E];
#pragma unroll
  for (int e = 0; e < CPL; e += 4) {
    const float4 c = ah.u[J % 3][e / 4];
    st.w[e] = fmaf(d, c.x, st.w[e]);
    st.w[e + 1] = fmaf(d, c.y, st.w[e + 1]);
    st.w[e + 2] = fmaf(d, c.z, st.w[e + 2]);
    st.w[e + 3] = fmaf(d, c.w, st.w[e + 3]);
  }
  if constexpr (CORR) {
    // W0_j - qhat_j, the same on every lane of the row
    const float dk = row_bcast<O>(st.w0[E]) - qh;
#pragma unroll
    for (int e = 0; e < CPL; e += 4) {
      st.corr[e] = fmaf(dk, pj[e / 4].x, st.corr[e]);
      st.corr[e + 1] = fmaf(dk, pj[e / 4].y, st.corr[e + 1]);
      st.corr[e + 2] = fmaf(dk, pj[e / 4].z, st.corr[e + 2]);
      st.corr[e + 3] = fmaf(dk, pj[e / 4].w, st.corr[e + 3]);
    }
  }
}

template <int B, int G, bool CORR, int... J>
__device__ __forceinline__ void gptq_steps(RowState<B / LPR>& st, Ahead<B / LPR>& ah,
                                           const StepCtx& cx, std::integer_sequence<int, J...>) {
  (gptq_step<B, G, CORR, J>(st, ah, cx), ...);
}

// 16 lanes per matrix row, each holding B/16 consecutive columns of the block.
// Per column: the current weight of column j is broadcast from the owning lane,
// every lane rounds it (same result), and every lane applies the feedback to its
// own columns (the LDS copy of U is zero on and below the diagonal, so no masks).
// A launch takes nblk (1 or 2) consecutive blocks.  The feedback product covers the
// columns before the launch; the second block's feedback from the first, D_1 P[1, 2]
// (D_1 = W0 - Qhat of the first block's columns), is accumulated column by column while
// the first block is quantized (P[1, 2] in LDS next to U_11).
// NBLK: the most blocks a launch takes (2 where the second block's state fits the registers
// next to the first's, else 1).
template <int B, int G, int NBLK>
__global__ __launch_bounds__(CTHREADS) void gptq_block_kernel(ColArgs a, int64_t j0) {
  constexpr int CPL = B / LPR;
  __shared__ __attribute__((aligned(16))) float Cb[B * B];
  __shared__ float Ri[B];
  __shared__ __attribute__((aligned(16))) float Pb[NBLK > 1 ? B * B : 4];
  const int t = threadIdx.x;
  const int q = t % LPR, rl = t / LPR;
  const int64_t r = (int64_t)blockIdx.x * RPW + rl;
  const bool live = r < a.out;
  const int64_t ypitch = (int64_t)a.nblk * B;
  // feedback into the current block from the launch's earlier block (zero for the first)
  float corr[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) corr[e] = 0.f;

  const int nblk = NBLK > 1 ? a.nblk : 1;
#pragma unroll 1
  for (int b = 0; b < nblk; ++b) {
    const int64_t jb = j0 + (int64_t)b * B;
    // the first of two blocks also forms the second's feedback from its own columns
    const bool corr_blk = NBLK > 1 && b + 1 < nblk;
    // All global loads first: U_JJ (and P[1, 2]), its diagonal, this row's starting weights,
    // feedback slices and dead flags.
    constexpr int NIT = B * B / 4 / CTHREADS;
    float4 uv[NIT], pv[NBLK > 1 ? NIT : 1];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = t + CTHREADS * it, i = idx / (B / 4), c = 4 * (idx % (B / 4));
      uv[it] = *(const float4*)(a.U + (jb + i) * a.in + jb + c);
    }
    if constexpr (NBLK > 1) {
      // P rows jb .. jb + B, columns jb + B .. jb + 2B (F above the next diagonal block);
      // read out of range (as 0, no branch around the loads) when there is no next block
      const __amdgpu_buffer_rsrc_t rp = rsrc(a.U + jb * a.in + jb + B);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = t + CTHREADS * it, i = idx / (B / 4), c = 4 * (idx % (B / 4));
        pv[it] = bload4(rp, corr_blk ? (int)((i * a.in + c) * 4) : OOB);
      }
    }
    const int td = t < B ? t : B - 1;
    const float udiag = a.U[(jb + td) * a.in + jb + td];
    RowState<CPL> st;
    const int64_t col = jb + CPL * q;
    float4 w0v[CPL / 4], yv[CPL / 4][YSLOTS];
    uint32_t dv[CPL / 4];
    // descriptor bases are per workgroup; the row goes into the lane's offset (r0 = first row)
    const int64_t r0 = (int64_t)blockIdx.x * RPW;
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.W + r0 * a.in + jb);
#pragma unroll
    for (int e = 0; e < CPL; e += 4) {
      w0v[e / 4] = bload4(rw, live ? (int)(((r - r0) * a.in + CPL * q + e) * 4) : OOB);
      dv[e / 4] = *(const uint32_t*)(a.dead + col + e);
      const int yoff = live ? (int)((r * ypitch + b * B + CPL * q + e) * 4) : OOB;
#pragma unroll
      for (int sp = 0; sp < YSLOTS; ++sp)
        yv[e / 4][sp] = bload4(rsrc(a.Y + sp * a.ystride), sp < a.nsplit ? yoff : OOB);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the previous block's readers of Cb and Ri are done
    if (b > 0) __syncthreads();

    // LDS copy of U_JJ, chunk-interleaved: columns [CPL q + 4 h, +4) of row i sit at
    // i * B + 4 (LPR h + q), so the 16 lanes of a row read 256 contiguous bytes per chunk;
    // entries on and below the diagonal are zeroed.  Ri = 1 / diag(U_JJ).
    if (t < B) Ri[t] = 1.0f / udiag;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = t + CTHREADS * it, i = idx / (B / 4), c = 4 * (idx % (B / 4));
      float4 v = uv[it];
      v.x = c + 0 > i ? v.x : 0.0f;
      v.y = c + 1 > i ? v.y : 0.0f;
      v.z = c + 2 > i ? v.z : 0.0f;
      v.w = c + 3 > i ? v.w : 0.0f;
      const int qq = c / CPL, hh = (c % CPL) / 4;
      *(float4*)(Cb + i * B + 4 * (LPR * hh + qq)) = v;
      if constexpr (NBLK > 1) *(float4*)(Pb + i * B + 4 * (LPR * hh + qq)) = pv[it];
    }

#pragma unroll
    for (int e = 0; e < CPL; e += 4) {
      float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int sp = 0; sp < YSLOTS; ++sp) {
        y.x += yv[e / 4][sp].x; y.y += yv[e / 4][sp].y; y.z += yv[e / 4][sp].z; y.w += yv[e / 4][sp].w;
      }
      const float4 w0 = w0v[e / 4];
      const uint32_t dd = dv[e / 4];
      st.w0[e] = (dd & 0xffu) ? 0.f : w0.x;
      st.w0[e + 1] = (dd & 0xff00u) ? 0.f : w0.y;
      st.w0[e + 2] = (dd & 0xff0000u) ? 0.f : w0.z;
      st.w0[e + 3] = (dd & 0xff000000u) ? 0.f : w0.w;
      st.w[e] = st.w0[e] + y.x + corr[e];
      st.w[e + 1] = st.w0[e + 1] + y.y + corr[e + 1];
      st.w[e + 2] = st.w0[e + 2] + y.z + corr[e + 2];
      st.w[e + 3] = st.w0[e + 3] + y.w + corr[e + 3];
      st.el[e] = st.el[e + 1] = st.el[e + 2] = st.el[e + 3] = 0.f;
      st.corr[e] = st.corr[e + 1] = st.corr[e + 2] = st.corr[e + 3] = 0.f;
      st.dl[e] = st.dl[e + 1] = st.dl[e + 2] = st.dl[e + 3] = 0.f;
      st.ql[e] = st.ql[e + 1] = st.ql[e + 2] = st.ql[e + 3] = 0.f;
    }
    st.s = 1.0f; st.inv = 1.0f; st.z = 0.0f;
    if constexpr (G == 0) {  // one group per row: grid taken from the original row beforehand
      if (live) {
        st.s = a.scales[r];
        st.inv = 1.0f / st.s;
        st.z = (float)a.zeros[r];
      }
    }
    __syncthreads();

    StepCtx cx{Cb, Pb, q, live, r, jb, &a};
    Ahead<CPL> ah;
#pragma unroll
    for (int i = 0; i < CPL; ++i) ah.ri[i] = Ri[LPR * i + q];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < CPL; e += 4) ah.u[jj][e / 4] = *(const float4*)(Cb + jj * B + 4 * q + LPR * e);
    if (NBLK > 1 && corr_blk) {
      gptq_steps<B, G, true>(st, ah, cx, std::make_integer_sequence<int, B>{});
#pragma unroll
      for (int e = 0; e < CPL; ++e) corr[e] = st.corr[e];
    } else {
      gptq_steps<B, G, false>(st, ah, cx, std::make_integer_sequence<int, B>{});
    }

    // Pack the row's B codes into bits * B / 32 whole words starting at word jb * bits / 32.
    // Lane q's CPL codes form one field of CPL * bits <= 32 bits at bit CPL * bits * q of the
    // row's code stream; word w (bits [32 w, 32 w + 32)) is gathered from the fields of the at
    // most five lanes that reach into it, placed in a 64-bit window 32 bits up so that every
    // shift is non-negative.
    uint32_t f = 0;
#pragma unroll
    for (int e = 0; e < CPL; ++e) f |= (uint32_t)st.ql[e] << (e * a.bits);
    const int fbits = CPL * a.bits;
    const int qa = (32 * q) / fbits;
    uint32_t fk[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) fk[k] = __shfl(f, qa + k < LPR ? qa + k : LPR - 1, LPR);
    uint64_t word = 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int off = (qa + k) * fbits - 32 * q;
      const bool use = qa + k < LPR && off < 32;
      word |= (uint64_t)(use ? fk[k] : 0u) << (use ? off + 32 : 0);
    }
    if (live) {
      const int64_t wpr = a.in * a.bits / 32;
      if (a.packed && q < a.bits * B / 32)
        a.packed[r * wpr + jb * a.bits / 32 + q] = (uint32_t)(word >> 32);
      if (a.codes) {
#pragma unroll
        for (int e = 0; e < CPL; e += 4)
          *(uint32_t*)(a.codes + r * a.in + col + e) =
              (uint32_t)st.ql[e] | ((uint32_t)st.ql[e + 1] << 8) | ((uint32_t)st.ql[e + 2] << 16) |
              ((uint32_t)st.ql[e + 3] << 24);
      }
      // errors replace the processed weights; W0 - qhat goes to D
#pragma unroll
      for (int e = 0; e < CPL; e += 4) {
        *(float4*)(a.W + r * a.in + col + e) = make_float4(st.el[e], st.el[e + 1], st.el[e + 2], st.el[e + 3]);
        *(float4*)(a.D + r * a.in + col + e) = make_float4(st.dl[e], st.dl[e + 1], st.dl[e + 2], st.dl[e + 3]);
      }
    }

  }
}

// |d|^2.4 in fp32 from the hardware base-2 log and exponential (0 for d = 0)
__device__ __forceinline__ float pow24(float d) {
  return __builtin_amdgcn_exp2f(2.4f * __builtin_amdgcn_logf(d));
}

// One (row) group spanning the whole row: grid from the original row (dead columns zeroed),
// one workgroup per row.  With clip, the grid of the shrunk range [p xmin, p xmax] for
// p = 1 - i/100, i < 80, with the smallest sum |s (q - z) - w|^2.4 over the row (the first
// such p on equal sums; each thread sums its terms in fp32, the threads' sums are added in
// fp64).  The row is staged in LDS when it fits (rows_in_lds).
constexpr int CLIP_CANDIDATES = 80;
__global__ __launch_bounds__(256) void row_grid_kernel(const float* __restrict__ W, int64_t in,
                                                       const uint8_t* __restrict__ dead, float maxq,
                                                       float* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros, int clip,
                                                       int rows_in_lds) {
  extern __shared__ float rowbuf[];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;
  const float* row = W + r * in;
  float mn = 0.f, mx = 0.f;
#pragma unroll 4
  for (int64_t c = t; c < in; c += 256) {
    const float v = dead[c] ? 0.f : row[c];
    if (rows_in_lds) rowbuf[c] = v;
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  __shared__ float smn[256], smx[256];
  __shared__ double sred[4];
  smn[t] = mn;
  smx[t] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      smn[t] = fminf(smn[t], smn[t + w]);
      smx[t] = fmaxf(smx[t], smx[t + w]);
    }
    __syncthreads();
  }
  const float xmin0 = smn[0], xmax0 = smx[0];
  if (!clip) {
    if (t == 0) {
      float s = (xmax0 - xmin0) / maxq;
      if (xmax0 == xmin0) s = 1.0f;
      scales[r] = s;
      zeros[r] = (uint8_t)rintf(-xmin0 / s);
    }
    return;
  }
  double best = INFINITY;
  float best_s = 1.0f, best_z = 0.0f;
  for (int i = 0; i < CLIP_CANDIDATES; ++i) {
    const double p = 1.0 - i / 100.0;
    const float xmin = (float)(p * xmin0), xmax = (float)(p * xmax0);
    float s = (xmax - xmin) / maxq;
    if (xmax == xmin) s = 1.0f;
    const float z = rintf(-xmin / s), inv = 1.0f / s;
    float ef = 0.0f;
#pragma unroll 4
    for (int64_t c = t; c < in; c += 256) {
      const float w = rows_in_lds ? rowbuf[c] : (dead[c] ? 0.f : row[c]);
      const float q = __builtin_amdgcn_fmed3f(rintf(w * inv) + z, 0.0f, maxq);
      ef += pow24(fabsf(s * (q - z) - w));
    }
    double e = (double)ef;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o);
    if ((t & 63) == 0) sred[t >> 6] = e;
    __syncthreads();
    if (t == 0) {
      const double tot = (sred[0] + sred[1]) + (sred[2] + sred[3]);
      if (tot < best) {
        best = tot;
        best_s = s;
        best_z = z;
      }
    }
    __syncthreads();
  }
  if (t == 0) {
    scales[r] = best_s;
    zeros[r] = (uint8_t)best_z;
  }
}

// act_order: column i's rank by descending diag(H) (a zero diagonal counts as 1, equal values
// by index), perm[rank] = i, invperm[i] = rank.  A NaN diagonal counts as -inf, so the order
// stays total and the ranks a permutation.  Three steps: the keys; partial ranks of 256
// columns against a 1024-key chunk per workgroup (atomically added); perm from the ranks.
__device__ __forceinline__ float act_key(float v) {
  return v == 0.f ? 1.f : (v != v ? -INFINITY : v);
}

__global__ __launch_bounds__(256) void act_keys_kernel(const float* __restrict__ H, int64_t n,
                                                       float* __restrict__ key,
                                                       int32_t* __restrict__ rank) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    key[i] = act_key(H[i * n + i]);
    rank[i] = 0;
  }
}

constexpr int RCHUNK = 1024;
__global__ __launch_bounds__(256) void act_rank_kernel(const float* __restrict__ key, int64_t n,
                                                       int32_t* __restrict__ rank) {
  __shared__ __attribute__((aligned(16))) float kc[RCHUNK];
  const int t = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * 256 + t;
  const int64_t j0 = (int64_t)blockIdx.y * RCHUNK;
#pragma unroll
  for (int k = t; k < RCHUNK; k += 256) {
    const int64_t j = j0 + k;
    // past the end: -inf with an index above every i, so it never outranks anything
    kc[k] = j < n ? key[j] : -INFINITY;
  }
  __syncthreads();
  if (i >= n) return;
  const float di = key[i];
  int cnt = 0;
  const int64_t m = min((int64_t)RCHUNK, n - j0);
  if (j0 + m <= i) {
    // every key of the chunk has a smaller index, so ties count (the chunk is full here:
    // only the last chunk is short, and it ends at n > i)
#pragma unroll 8
    for (int k = 0; k < RCHUNK; k += 4) {
      const float4 v = *(const float4*)(kc + k);
      cnt += (v.x >= di) + (v.y >= di) + (v.z >= di) + (v.w >= di);
    }
  } else if (j0 > i) {
    // every key has a larger index, so ties do not count (padding keys are -inf: never greater)
#pragma unroll 8
    for (int k = 0; k < RCHUNK; k += 4) {
      const float4 v = *(const float4*)(kc + k);
      cnt += (v.x > di) + (v.y > di) + (v.z > di) + (v.w > di);
    }
  } else {
    for (int k = 0; k < m; ++k) {
      const float dj = kc[k];
      cnt += (dj > di) | ((dj == di) & (j0 + k < i));
    }
  }
  atomicAdd(rank + i, cnt);
}

__global__ __launch_bounds__(256) void act_perm_kernel(const int32_t* __restrict__ rank, int64_t n,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ invperm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    perm[rank[i]] = (int32_t)i;
    invperm[i] = rank[i];
  }
}

// dst[r][c] = src[rows ? rows[r] : r][idx[c]], c < n: one workgroup per row, the source row
// staged in LDS (n * sizeof(T) bytes of dynamic LDS).  src and dst must not overlap.
template <typename T>
__global__ __launch_bounds__(256) void gather_cols_kernel(const T* __restrict__ src,
                                                          T* __restrict__ dst, int64_t n,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ rows) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gbuf[];
  T* row = (T*)gbuf;
  const int64_t r = blockIdx.x;
  const int64_t sr = rows ? rows[r] : r;
  const int t = threadIdx.x;
#pragma unroll 4
  for (int64_t c = t; c < n; c += 256) row[c] = src[sr * n + c];
  __syncthreads();
#pragma unroll 4
  for (int64_t c = t; c < n; c += 256) dst[r * n + c] = row[idx[c]];
}

// Packs rows of codes (column order) into bits * in / 32 words per row: word w holds bits
// [32 w, 32 w + 32) of the row's stream, i.e. codes c0 .. c0 + 16 at most, gathered in a
// 64-bit window 8 bits up so that every shift is non-negative.
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint8_t* __restrict__ codes,
                                                        int64_t out, int64_t in, int bits,
                                                        uint32_t* __restrict__ packed) {
  const int64_t words = in * bits / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= out * words) return;
  const int64_t r = idx / words, w = idx % words;
  const int64_t bit0 = 32 * w, c0 = bit0 / bits;
  const uint8_t* cr = codes + r * in;
  uint32_t v[17];
#pragma unroll
  for (int k = 0; k < 17; ++k) v[k] = cr[c0 + k < in ? c0 + k : in - 1];
  uint64_t acc = 0;
#pragma unroll
  for (int k = 0; k < 17; ++k) {
    const int64_t c = c0 + k, off = c * bits - bit0;
    const bool use = c < in && off < 32;
    acc |= (uint64_t)(use ? v[k] : 0u) << (use ? off + 8 : 0);
  }
  packed[r * words + w] = (uint32_t)(acc >> 8);
}

// sum of a[i] * b[i] over n elements into *red (fp64)
__global__ __launch_bounds__(256) void dot_kernel(const float* __restrict__ x,
                                                  const float* __restrict__ y, int64_t n,
                                                  double* __restrict__ red) {
  double s = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    s += (double)x[i] * (double)y[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) atomicAdd(red, s);
}

using ColKernel = void (*)(ColArgs, int64_t);

// The column kernel for block B and group G, and the most blocks it takes per launch.
ColKernel pick_kernel(int B, int G, int* nblk) {
  *nblk = 1;
  if (B == 64) {
    *nblk = 2;
    switch (G) {
      case 0: return gptq_block_kernel<64, 0, 2>;
      case 16: return gptq_block_kernel<64, 16, 2>;
      case 32: return gptq_block_kernel<64, 32, 2>;
      case 64: return gptq_block_kernel<64, 64, 2>;
    }
  } else if (B == 128) {
    switch (G) {
      case 0: *nblk = 2; return gptq_block_kernel<128, 0, 2>;
      case 16: return gptq_block_kernel<128, 16, 1>;
      case 32: return gptq_block_kernel<128, 32, 1>;
      case 64: return gptq_block_kernel<128, 64, 1>;
      case 128: *nblk = 2; return gptq_block_kernel<128, 128, 2>;
    }
  }
  return nullptr;
}

// dst[r][c] = src[rows ? rows[r] : r][idx[c]] without LDS staging (rows longer than 64 KB)
template <typename T>
__global__ __launch_bounds__(256) void gather_cols_direct_kernel(const T* __restrict__ src,
                                                                 T* __restrict__ dst, int64_t n,
                                                                 const int32_t* __restrict__ idx,
                                                                 const int32_t* __restrict__ rows) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (c >= n) return;
  const int64_t sr = rows ? rows[r] : r;
  dst[r * n + c] = src[sr * n + idx[c]];
}

// Largest row staged in LDS by the row kernels (bytes; rows longer than 16384 floats take
// the direct paths, which tests can force with 0).
size_t row_lds_max() {
  const int64_t v = testing_value(KQ_TESTING_ROW_LDS_BYTES, 65536);
  return (size_t)(v > 65536 ? 65536 : v);
}

template <typename T>
kq_status gather_cols(const T* src, T* dst, int64_t nrows, int64_t n, const int32_t* idx,
                      const int32_t* rows, hipStream_t s) {
  const size_t bytes = (size_t)n * sizeof(T);
  if (bytes <= row_lds_max()) {
    gather_cols_kernel<T><<<dim3((unsigned)nrows), dim3(256), bytes, s>>>(src, dst, n, idx, rows);
    KQ_LAUNCHED("gather_cols_kernel");
  } else {
    gather_cols_direct_kernel<T><<<dim3((unsigned)ceil_div(n, 256), (unsigned)nrows), dim3(256), 0,
                                   s>>>(src, dst, n, idx, rows);
    KQ_LAUNCHED("gather_cols_direct_kernel");
  }
  return KQ_OK;
}

struct Layout {
  size_t f, t, y, d, dead, scal, flag, tmp, perm, invperm, ptmp, ctmp, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout layout(int64_t out, int64_t in, int B, bool with_loss, bool act_order) {
  Layout L;
  size_t o = 0;
  L.f = o;    o = align256(o + (size_t)in * in * sizeof(float));
  L.t = o;    o = align256(o + (size_t)in * 128 * sizeof(float));
  L.y = o;    o = align256(o + (size_t)y_slots(out, B) * out * 2 * B * sizeof(float));
  L.d = o;    o = align256(o + (size_t)out * in * sizeof(float));
  L.dead = o; o = align256(o + (size_t)in);
  L.scal = o; o = align256(o + 8 * sizeof(double));
  L.flag = o; o = align256(o + 4 * sizeof(int));
  L.tmp = o;  if (with_loss) o = align256(o + (size_t)out * in * sizeof(float));
  // act_order: the permutation and its inverse, a staging matrix and the permuted codes
  L.perm = L.invperm = L.ptmp = L.ctmp = o;
  if (act_order) {
    L.perm = o;    o = align256(o + (size_t)in * sizeof(int32_t));
    L.invperm = o; o = align256(o + (size_t)in * sizeof(int32_t));
    L.ptmp = o;    o = align256(o + (size_t)out * in * sizeof(float));
    L.ctmp = o;    o = align256(o + (size_t)out * in);
  }
  L.total = o;
  return L;
}

kq_status check_params(const kq_quant_params* p, int64_t out, int64_t in) {
  if (!p) return fail(KQ_EINVAL, "kq_quantize_layer: params is NULL");
  if (p->bits < 2 || p->bits > 4) return fail(KQ_EINVAL, "bits must be 2, 3 or 4 (got %d)", p->bits);
  if (p->asym != 1) return fail(KQ_ENOTIMPL, "only the asymmetric grid (asym = 1) is implemented");
  if (p->act_order != 0 && p->act_order != 1) return fail(KQ_EINVAL, "act_order must be 0 or 1");
  if (p->w_clip != 0 && p->w_clip != 1) return fail(KQ_EINVAL, "w_clip must be 0 or 1");
  if (!(p->damp >= 0.f) || !isfinite(p->damp)) return fail(KQ_EINVAL, "damp must be >= 0");
  if (p->block != 64 && p->block != 128) return fail(KQ_EINVAL, "block must be 64 or 128");
  if (out < 1 || in < 1 || in > (1 << 30) || out > (1 << 22))
    return fail(KQ_ESHAPE, "bad layer shape");
  if (in % 32 != 0) return fail(KQ_ESHAPE, "in must be a multiple of 32");
  if (in % p->block != 0) return fail(KQ_ESHAPE, "in must be a multiple of block");
  if (p->group <= 0 || in % p->group != 0)
    return fail(KQ_ESHAPE, "group must be positive and divide in");
  if (p->group != in && (p->group > p->block || p->block % p->group != 0 ||
                         (p->group != 16 && p->group != 32 && p->group != 64 && p->group != 128)))
    return fail(KQ_ESHAPE, "group must be in {16, 32, 64, 128} dividing block, or equal to in");
  if ((p->act_order || p->w_clip) && p->group != in)
    return fail(KQ_ENOTIMPL, "act_order and w_clip take one grid per row (group == in)");
  return KQ_OK;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_quantize_layer_workspace(const kq_quant_params* p, int64_t out, int64_t in,
                                                 int with_loss, size_t* bytes) {
  using namespace kq;
  if (!bytes) return fail(KQ_EINVAL, "kq_quantize_layer_workspace: bytes is NULL");
  KQ_TRY(check_params(p, out, in));
  *bytes = layout(out, in, p->block, with_loss != 0, p->act_order != 0).total;
  return KQ_OK;
}

namespace kq {
namespace {

// Status and losses of an asynchronous call, written when its work has run.
__global__ void quantize_finish_kernel(const double* __restrict__ scal, const int* __restrict__ flag,
                                       double* __restrict__ loss_dev, int* __restrict__ status_dev) {
  if (threadIdx.x == 0) {
    if (loss_dev) {
      loss_dev[0] = scal[1];
      loss_dev[1] = scal[2];
    }
    *status_dev = flag[0] ? (int)KQ_ENOTSPD : (int)KQ_OK;
  }
}

// The quantizer.  Synchronous (status_dev == NULL): losses to the host loss_opt, the status
// returned after a stream synchronization.  Asynchronous: losses to the device loss_dev, the
// status to the device status_dev, nothing waited for.
kq_status quantize_layer(const kq_quant_params* p, float* W_rot, const float* HX_rot,
                         const float* HG_rot, int64_t out, int64_t in, uint32_t* packed,
                         float* scales, uint8_t* zeros, uint8_t* codes_opt, double* loss_opt,
                         void* ws, size_t ws_bytes, void* stream, double* loss_dev = nullptr,
                         int* status_dev = nullptr) {
  KQ_TRY(check_params(p, out, in));
  if (!W_rot || !HX_rot || !packed || !scales || !zeros)
    return fail(KQ_EINVAL, "kq_quantize_layer: NULL argument");
  const bool with_loss = loss_opt != nullptr || loss_dev != nullptr;
  const int B = p->block;
  const bool ao = p->act_order != 0, clip = p->w_clip != 0;
  // a group spanning the whole row (group == in > block, or any row grid with act_order or
  // w_clip) takes its grid from the original row
  const int G = p->group == in && (p->group > B || ao || clip) ? 0 : p->group;
  const Layout L = layout(out, in, B, with_loss, ao);
  if (!ws || ws_bytes < L.total)
    return fail(KQ_EWORKSPACE, "kq_quantize_layer: workspace of %zu bytes needed", L.total);
  int max_blk = 1;
  ColKernel kern = pick_kernel(B, G, &max_blk);
  if (!kern) return fail(KQ_ESHAPE, "no column kernel for block %d group %d", B, G);
  hipStream_t s = as_stream(stream);
  char* base = (char*)ws;
  float* F = (float*)(base + L.f);
  float* T = (float*)(base + L.t);
  float* Y = (float*)(base + L.y);
  float* Dm = (float*)(base + L.d);
  uint8_t* dead = (uint8_t*)(base + L.dead);
  double* scal = (double*)(base + L.scal);
  int* flag = (int*)(base + L.flag);

  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* invperm = (int32_t*)(base + L.invperm);
  float* Ptmp = (float*)(base + L.ptmp);
  uint8_t* ctmp = (uint8_t*)(base + L.ctmp);

  KQ_TRY(fill_u32((uint32_t*)scal, 16, 0u, s));
  KQ_TRY(fill_u32((uint32_t*)flag, 4, 0u, s));
  if (ao) {
    // act_order: F = H~_X[perm][perm] and W~ <- W~[:, perm]; GPTQ then runs in that order
    float* keys = Ptmp;   // free until W~ is gathered
    int32_t* rank = invperm;
    const unsigned cb = (unsigned)ceil_div(in, 256);
    act_keys_kernel<<<dim3(cb), dim3(256), 0, s>>>(HX_rot, in, keys, rank);
    KQ_LAUNCHED("act_keys_kernel");
    act_rank_kernel<<<dim3(cb, (unsigned)ceil_div(in, RCHUNK)), dim3(256), 0, s>>>(keys, in, rank);
    KQ_LAUNCHED("act_rank_kernel");
    act_perm_kernel<<<dim3(cb), dim3(256), 0, s>>>(rank, in, perm, invperm);
    KQ_LAUNCHED("act_perm_kernel");
    KQ_TRY(gather_cols<float>(HX_rot, F, in, in, perm, perm, s));
    KQ_TRY(gather_cols<float>(W_rot, Ptmp, out, in, perm, nullptr, s));
  }
  // the weights GPTQ works on (and leaves its errors in): W~, or its permuted copy
  float* Wq = ao ? Ptmp : W_rot;
  KQ_TRY(damp_and_factor(ao ? nullptr : HX_rot, F, T, dead, scal, flag, in, p->damp, B, s));

  ColArgs a;
  a.W = Wq; a.out = out; a.in = in; a.Y = Y; a.D = Dm; a.U = F; a.dead = dead;
  a.nsplit = 0; a.ystride = out * B; a.nblk = 1;
  a.bits = p->bits; a.maxq = (float)((1 << p->bits) - 1);
  a.ngroups = in / p->group; a.scales = scales; a.zeros = zeros;
  a.packed = ao ? nullptr : packed; a.codes = ao ? ctmp : codes_opt;
  if (G == 0) {
    const int lds_row = clip && in * sizeof(float) <= row_lds_max();
    row_grid_kernel<<<dim3((unsigned)out), dim3(256), lds_row ? in * sizeof(float) : 0, s>>>(
        Wq, in, dead, a.maxq, scales, zeros, clip ? 1 : 0, lds_row);
    KQ_LAUNCHED("row_grid_kernel");
  }
  const int cus = device_cu_count();
  const unsigned col_grid = (unsigned)ceil_div(out, RPW);
  // two blocks per launch where the kernel takes them (it forms the second block's feedback
  // from the first); a last odd block alone
  for (int64_t j0 = 0; j0 < in; j0 += (int64_t)a.nblk * B) {
    a.nblk = max_blk > 1 && j0 + 2 * B <= in ? 2 : 1;
    const int64_t N = (int64_t)a.nblk * B;
    a.ystride = out * N;
    a.nsplit = 0;
    if (j0 > 0) {
      GemmArgs g{};
      g.M = out; g.N = N; g.K = j0;
      g.A = Dm; g.lda = in; g.transA = false;
      g.B = F + j0; g.ldb = in; g.transB = false;
      g.C = Y; g.ldc = N; g.alpha = 1.0f; g.accumulate = false; g.upper_only = false;
      // one workgroup per CU (the product keeps a 128 KB LDS ring): split K where whole
      // rounds of workgroups then cover the GPU better, down to one 32-deep stage per split;
      // each split stores its own slice (out x N, as many as the workspace holds), which the
      // column kernel sums
      const int64_t cap = std::min<int64_t>(YSLOTS, 2 * y_slots(out, B) / a.nblk);
      g.split_k = (int)feedback_splits(out, N, ceil_div(j0, 32), cap, cus);
      g.partial_stride = out * N;
      g.splits_used = &a.nsplit;
      KQ_TRY(gemm_f32(g, s));
    }
    kern<<<dim3(col_grid), dim3(CTHREADS), 0, s>>>(a, j0);
    KQ_LAUNCHED("gptq_block_kernel");
  }
  // W~ - Qhat in the original column order, for the losses
  const float* dW = Dm;
  if (ao) {
    // back to the original column order: errors into W_rot, W~ - Qhat (for the losses) into
    // the staging buffer, codes (into D's memory when the caller keeps none), packing
    KQ_TRY(gather_cols<float>(Ptmp, W_rot, out, in, invperm, nullptr, s));
    if (with_loss) {
      KQ_TRY(gather_cols<float>(Dm, Ptmp, out, in, invperm, nullptr, s));
      dW = Ptmp;
    }
    uint8_t* cout = codes_opt ? codes_opt : (uint8_t*)Dm;
    KQ_TRY(gather_cols<uint8_t>(ctmp, cout, out, in, invperm, nullptr, s));
    const int64_t nw = out * (in * p->bits / 32);
    pack_rows_kernel<<<dim3((unsigned)ceil_div(nw, 256)), dim3(256), 0, s>>>(cout, out, in, p->bits,
                                                                            packed);
    KQ_LAUNCHED("pack_rows_kernel");
  }

  if (with_loss) {
    // dW = W~ - Qhat
    float* tmp = (float*)(base + L.tmp);
    // predicted loss  sum_j e_j^T H~_G e_j
    if (HG_rot) {
      GemmArgs r{};
      r.M = out; r.N = out; r.K = in;
      r.A = W_rot; r.lda = in; r.B = W_rot; r.ldb = in; r.transB = true;
      r.alpha = 1.0f; r.split_k = 1; r.D = HG_rot; r.ldd = out; r.red = scal + 2;
      KQ_TRY(gemm_f32(r, s));
    } else {
      dot_kernel<<<dim3(1024), dim3(256), 0, s>>>(W_rot, W_rot, out * in, scal + 2);
      KQ_LAUNCHED("dot_kernel");
    }
    // tmp = dW H~_X (undamped), direct loss sum (tmp dW^T) .* H~_G
    GemmArgs h{};
    h.M = out; h.N = in; h.K = in;
    h.A = dW; h.lda = in; h.B = HX_rot; h.ldb = in; h.C = tmp; h.ldc = in;
    h.alpha = 1.0f; h.split_k = 1;
    KQ_TRY(gemm_f32(h, s));
    if (HG_rot) {
      GemmArgs r{};
      r.M = out; r.N = out; r.K = in;
      r.A = tmp; r.lda = in; r.B = dW; r.ldb = in; r.transB = true;
      r.alpha = 1.0f; r.split_k = 1; r.D = HG_rot; r.ldd = out; r.red = scal + 1;
      KQ_TRY(gemm_f32(r, s));
    } else {
      dot_kernel<<<dim3(1024), dim3(256), 0, s>>>(tmp, dW, out * in, scal + 1);
      KQ_LAUNCHED("dot_kernel");
    }
  }
  if (status_dev) {
    quantize_finish_kernel<<<dim3(1), dim3(64), 0, s>>>(scal, flag, loss_dev, status_dev);
    KQ_LAUNCHED("quantize_finish_kernel");
    return KQ_OK;
  }
  double host_scal[3] = {0, 0, 0};
  int host_flag = 0;
  KQ_HIP(hipMemcpyAsync(host_scal, scal, sizeof(host_scal), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  if (with_loss) {
    loss_opt[0] = host_scal[1];
    loss_opt[1] = host_scal[2];
  }
  if (host_flag) return fail(KQ_ENOTSPD, "kq_quantize_layer: damped H_X is not positive definite");
  return KQ_OK;
}

// Workspace of kq_quantize_layer_noalloc: one copy per GPU, held until the process ends.  Host
// code never names it directly (its host-side name is no device address): the device address
// comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t NOALLOC_SCRATCH_BYTES = KQ_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

kq_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  KQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(KQ_ENOTIMPL, "kq_quantize_layer_noalloc: device index %d beyond %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    KQ_HIP(hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)));
    if (!a) return fail(KQ_EHIP, "kq_quantize_layer_noalloc: no device address for the scratch");
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return KQ_OK;
}

}  // namespace
}  // namespace kq

extern "C" kq_status kq_quantize_layer(const kq_quant_params* p, float* W_rot, const float* HX_rot,
                                       const float* HG_rot, int64_t out, int64_t in,
                                       uint32_t* packed, float* scales, uint8_t* zeros,
                                       uint8_t* codes_opt, double* loss_opt, void* ws,
                                       size_t ws_bytes, void* stream) {
  return kq::quantize_layer(p, W_rot, HX_rot, HG_rot, out, in, packed, scales, zeros, codes_opt,
                            loss_opt, ws, ws_bytes, stream);
}

extern "C" kq_status kq_quantize_layer_async(const kq_quant_params* p, float* W_rot,
                                             const float* HX_rot, const float* HG_rot,
                                             int64_t out, int64_t in, uint32_t* packed,
                                             float* scales, uint8_t* zeros, uint8_t* codes_opt,
                                             double* loss_dev_opt, int* status_dev, void* ws,
                                             size_t ws_bytes, void* stream) {
  if (!status_dev) return kq::fail(KQ_EINVAL, "kq_quantize_layer_async: status_dev is NULL");
  return kq::quantize_layer(p, W_rot, HX_rot, HG_rot, out, in, packed, scales, zeros, codes_opt,
                            nullptr, ws, ws_bytes, stream, loss_dev_opt, status_dev);
}

extern "C" kq_status kq_quantize_layer_noalloc(const kq_quant_params* p, float* W_rot,
                                               const float* HX_rot, const float* HG_rot,
                                               int64_t out, int64_t in, uint32_t* packed,
                                               float* scales, uint8_t* zeros, uint8_t* codes_opt,
                                               double* loss_opt, void* stream) {
  using namespace kq;
  KQ_TRY(check_params(p, out, in));
  const size_t need = layout(out, in, p->block, loss_opt != nullptr, p->act_order != 0).total;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(KQ_EWORKSPACE,
                "kq_quantize_layer_noalloc: this layer needs %zu bytes of workspace, more than the "
                "library's fixed %zu; use kq_quantize_layer with a workspace of its own",
                need, NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  KQ_TRY(scratch_of_current_device(&ws));
  return quantize_layer(p, W_rot, HX_rot, HG_rot, out, in, packed, scales, zeros, codes_opt,
                        loss_opt, ws, NOALLOC_SCRATCH_BYTES, stream);
}
