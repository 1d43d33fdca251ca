/*
 * kq.h -- C ABI of the KronQ per-layer quantization engine for AMD Instinct
 * MI355X (gfx950).
 *
 * What the engine computes, per linear layer (W is out x in, rows = output
 * channels; X is tokens x in calibration activations, G is tokens x out output
 * gradients):
 *   1. the Kronecker Hessian factors H_X = X^T X and H_G = G^T G
 *      (KronQ README, opening section: H ~ H_X (x) H_G; WaterKron and FlipFlop
 *      Hessian, Table 1, row "Marginal");
 *   2. the sensitivity tr(H_G) tr(H_X) that drives inter-layer bit allocation
 *      (KronQ README, opening section; KronQ arXiv abstract, point 2);
 *   3. bidirectional incoherence processing (BiIP): rescale plus randomized
 *      Hadamard rotation on the input and the output side (KronQ README,
 *      opening section and flags table; KronQ arXiv abstract, point 1);
 *   4. GPTQ error-feedback quantization through a damped Cholesky factor of
 *      H_X^-1, to packed 2/3/4-bit codes, minimizing tr(H_G dW H_X dW^T)
 *      (KronQ README, opening section and "Mapping paper results to flags");
 *   5. the per-sublayer bit allocation to an average bit budget.
 *
 * Conventions for every entry point:
 *   - Matrix arguments are row-major with the stated leading dimension (in
 *     elements).  Pointers are device pointers (memory from hipMalloc or a
 *     PyTorch CUDA/HIP tensor) unless the argument says "host".
 *   - The caller owns every buffer.  Entry points never keep a pointer after
 *     they return and never free caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued on it and the call returns without waiting, except where an
 *     entry point says it synchronizes.
 *   - All argument checks run on the host before anything is enqueued.  A
 *     non-OK status means nothing was enqueued, except KQ_EHIP (a launch or
 *     runtime call failed) and KQ_ENOTSPD (reported after the work ran).
 *   - kq_last_error() returns a thread-local message for the last non-OK
 *     status of the calling thread.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kq_status {
  KQ_OK = 0,
  KQ_EINVAL = 1,      /* NULL pointer, bad enum value, bits outside {2,3,4}, ... */
  KQ_ESHAPE = 2,      /* sizes that the operation does not accept */
  KQ_ENOTSPD = 3,     /* damped H_X has a non-positive pivot (no Cholesky factor) */
  KQ_EWORKSPACE = 4,  /* workspace NULL or smaller than the queried size */
  KQ_ENOTIMPL = 5,    /* option not implemented */
  KQ_EHIP = 6         /* a HIP runtime call or kernel launch failed */
} kq_status;

/* Incoherence-processing modes (KronQ README, "Mapping paper results to flags":
 * --incoh_mode {full, no_rescale, su_only, sv_only}; the one-sided modes are
 * read here as input-side-only and output-side-only processing). */
enum {
  KQ_BIIP_FULL = 0,       /* rescale + rotate, both sides */
  KQ_BIIP_NO_RESCALE = 1, /* rotate both sides, no rescale */
  KQ_BIIP_IN_ONLY = 2,    /* rescale + rotate the input side only */
  KQ_BIIP_OUT_ONLY = 3    /* rescale + rotate the output side only */
};

/* Quantizer parameters (KronQ README flags: --w_bits, --w_groupsize, --w_asym;
 * GPTQ's lazy block size and damping).  Defaults: bits 2, group 128,
 * block 128, damp 0.01, asym 1, act_order 0. */
typedef struct kq_quant_params {
  int bits;       /* 2, 3 or 4 */
  int group;      /* columns per (row, group) scale/zero; 0 < group, in % group == 0 */
  int block;      /* GPTQ block width: 64 or 128; block % group == 0 or group % block == 0 */
  float damp;     /* lambda = damp * mean(diag H_X), damp >= 0 */
  int asym;       /* must be 1 (asymmetric min-max grid) */
  int act_order;  /* 0: natural column order; 1: descending diag(H~_X) (needs group == in) */
  int w_clip;     /* 0: min-max grid; 1: clip-ratio search per row (needs group == in) */
} kq_quant_params;

/* Library version: major * 10000 + minor * 100 + patch. */
int kq_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char* kq_last_error(void);

/*
 * kq_accumulate_hessian -- one Kronecker factor, H = A^T A or H += A^T A.
 *
 * Follows: KronQ README, opening section (K-FAC factorization H ~ H_X (x) H_G);
 * WaterKron and FlipFlop Hessian, Table 1, "Marginal" (input factor E[x x^T],
 * output factor E[g g^T]).  Sums are not normalized by the token count.
 *
 *   A_bf16      device, bf16 bit patterns, T x n, row-major, leading dim lda >= n
 *               (token-major: row t holds token t's n channels).  lda must be a
 *               multiple of 8 and A 16-byte aligned.
 *   T           tokens (>= 0; T = 0 leaves H = 0, or unchanged when accumulating)
 *   n           channels (1 <= n); H is n x n
 *   H           device fp32, n x n, leading dim ldh >= n.  On return H is the full
 *               symmetric matrix (both triangles written).
 *   accumulate  0: H = A^T A.  1: H += A^T A (H must hold a symmetric matrix).
 * Products of bf16 values are exact in fp32; accumulation is fp32.
 * Layout note: a stream 4096 channels wide runs about 10 % faster with a row pitch that is
 * not a multiple of 8 KB (lda = 4104, say) than with lda = n; at 8192 and 28672 channels the
 * pitch makes no measurable difference.
 */
kq_status kq_accumulate_hessian(const uint16_t* A_bf16, int64_t T, int64_t n, int64_t lda,
                                float* H, int64_t ldh, int accumulate, void* stream);

/*
 * kq_sensitivity -- traces and the sensitivity s = tr(H_G) * tr(H_X).
 *
 * Follows: KronQ README, opening section (the per-sublayer bit widths are chosen from
 * the product of the two factors' traces); KronQ arXiv abstract, point 2.
 * Meant for the raw factors (before BiIP).
 *
 *   HX   device fp32, n_in x n_in (leading dim ldx); only the diagonal is read
 *   HG   device fp32, n_out x n_out (leading dim ldg); only the diagonal is read
 *   out3 host, 3 doubles: {tr H_X, tr H_G, tr H_G * tr H_X}; diagonals summed in fp64
 * Synchronizes `stream` before returning.  The result passes through a 24-byte buffer in
 * the library's device memory, one per GPU, so calls from several host threads take turns
 * (a process-wide lock); kq_sensitivity_async, with memory of the caller's, runs unserialized.
 */
kq_status kq_sensitivity(const float* HX, int64_t n_in, int64_t ldx, const float* HG,
                         int64_t n_out, int64_t ldg, double out3[3], void* stream);

/*
 * kq_sensitivity_async -- kq_sensitivity with its result left in device memory.
 *
 * Follows: the same passages as kq_sensitivity, and computes the same three values (the same
 * reduction order, so bit-identical results).  Enqueues one kernel on `stream` and returns
 * without synchronizing, so a caller that quantizes many layers in a row keeps the GPU busy
 * and reads all sensitivities after its own synchronization.
 *
 *   HX, HG    as for kq_sensitivity
 *   out3_dev  device, 3 doubles owned by the caller: {tr H_X, tr H_G, tr H_G * tr H_X},
 *             written when the kernel runs
 * Errors (NULL argument, bad sizes) are reported before anything is enqueued.
 */
kq_status kq_sensitivity_async(const float* HX, int64_t n_in, int64_t ldx, const float* HG,
                               int64_t n_out, int64_t ldg, double* out3_dev, void* stream);

/*
 * kq_biip_rotate -- bidirectional incoherence processing of one layer.
 *
 * Follows: KronQ README, opening section (the incoherence rotation and the rescale
 * are applied on the input side and on the output side) and flags table (--incoh_kernel had,
 * --alpha 0.25); KronQ arXiv abstract, point 1.
 * With D_in = diag(d_in), D_out = diag(d_out) and P = blockdiag(Had_b) diag(S) / sqrt(b)
 * (Sylvester Hadamard of order b in natural order, S the +-1 signs):
 *   d_in[i]  = (H_X[i,i] / sum_r W[r,i]^2) ^ alpha      (1 if either is 0)
 *   d_out[k] = (H_G[k,k] / sum_i W[k,i]^2) ^ alpha      (1 if either is 0)
 *   W~   = P_out D_out W D_in P_in^T
 *   H~_X = P_in D_in^-1 H_X D_in^-1 P_in^T
 *   H~_G = P_out D_out^-1 H_G D_out^-1 P_out^T
 * which leaves tr(H_G dW H_X dW^T) unchanged for dW mapped like W.
 *
 *   W_src, W_dst     device fp32, out x in, contiguous rows (ld = in); may alias
 *   HX_src, HX_dst   device fp32, in x in symmetric, contiguous; may alias
 *   HG_src, HG_dst   device fp32, out x out symmetric, contiguous; may alias.
 *                    May both be NULL only in mode KQ_BIIP_IN_ONLY.
 *   sign_in/out      device int8 +-1, lengths in / out (sign_out unused in IN_ONLY,
 *                    sign_in unused in OUT_ONLY)
 *   had_block_in/out Hadamard block per side: 0 = the largest power of 2 that
 *                    divides the size (KQ_ENOTIMPL when that exceeds 8192, the
 *                    largest block implemented); else 1 (no transform on that
 *                    side's rows) or a power of 2 in [4, 8192] dividing it
 *   alpha            rescale exponent (0.25 for weight-only KronQ)
 *   mode             KQ_BIIP_*
 *   d_in, d_out      device fp32 outputs, lengths in / out (1 where not rescaled)
 * Sizes: 1 <= in, out; in and out must be multiples of 4.
 */
kq_status kq_biip_rotate(const float* W_src, float* W_dst, int64_t out, int64_t in,
                         const float* HX_src, float* HX_dst, const float* HG_src, float* HG_dst,
                         const int8_t* sign_in, const int8_t* sign_out, int64_t had_block_in,
                         int64_t had_block_out, float alpha, int mode, float* d_in, float* d_out,
                         void* stream);

/*
 * kq_quantize_layer_workspace -- device workspace bytes kq_quantize_layer needs.
 *   with_loss: nonzero if the call will request losses.
 */
kq_status kq_quantize_layer_workspace(const kq_quant_params* p, int64_t out, int64_t in,
                                      int with_loss, size_t* bytes);

/*
 * kq_quantize_layer -- damp, factor and GPTQ-quantize a processed layer to packed codes.
 *
 * Follows: KronQ README, opening section (weight-only W2-W4, GPTQ-based with
 * the K-FAC objective tr(H_G dW H_X dW^T)) and flags table (GPTQ base
 * quantizer, --w_asym, --w_groupsize).  Steps:
 *   dead input channels (H~_X[i,i] == 0): diagonal set to 1, weight column zeroed;
 *   lambda = damp * mean(diag H~_X);  H_d = H~_X + lambda I;
 *   GPTQ column by column with U = chol_upper(H_d^-1): at each group's first
 *   column the (row, group) grid is taken from the current weights
 *   (xmin = min(0, min), xmax = max(0, max), s = (xmax - xmin) / (2^b - 1) or 1 if
 *   equal, z = rint(-xmin / s)); code q = clamp(rint(w / s) + z, 0, 2^b - 1)
 *   (round half to even); the rounding error is fed back into later columns.
 * Base-recipe options (KronQ README, "Reproduce from scratch": --act_order and --w_clip
 * with --w_groupsize -1; the pages name them without defining them), both for one grid
 * per row (group == in):
 *   act_order = 1: GPTQ visits the columns in descending order of diag(H~_X) (a dead
 *     channel's zero counts as 1; equal values keep index order).  Every output (codes,
 *     packed words, errors in W_rot, losses) is still in the original column order.
 *   w_clip = 1: the row's grid is the min-max grid of the shrunk range [p xmin, p xmax]
 *     for the p in {1 - i/100 : i = 0..79} with the smallest sum |qhat - w|^2.4 over the
 *     row (the first such p on equal sums; fp32 terms and per-thread sums, added in fp64).
 * Implementation: reverse-order Cholesky H_d = R R^T (R upper), U = R^-1 formed only
 * in its diagonal blocks, and the column recursion run 128 (or 64) columns at a time
 * with one matrix product per block for the feedback from earlier blocks
 * ((W~ - Qhat)[:, <J] R[<J, J] U_JJ, which equals -E[:, <J] U[<J, J]).
 *
 *   W_rot     device fp32, out x in (ld = in), the processed weights W~.  Clobbered:
 *             on return column j holds GPTQ's error e_j = (w_j - qhat_j) / U_jj
 *             (dead columns 0), so W~ - Qhat = E U.
 *   HX_rot    device fp32, in x in symmetric (ld = in), H~_X; not modified
 *   HG_rot    device fp32, out x out (ld = out), H~_G; used only for losses; may be NULL
 *             (identity)
 *   packed    device uint32, out x (in * bits / 32): row r's codes as one
 *             little-endian bitstream, code i at bits [bits*i, bits*i + bits)
 *   scales    device fp32, out x (in / group)
 *   zeros     device uint8, out x (in / group)
 *   codes_opt device uint8, out x in, or NULL
 *   loss_opt  host double[2] or NULL: {tr(H~_G dW H~_X dW^T), the same with H_d}
 *             (direct loss and GPTQ's predicted loss sum_j e_j^T H~_G e_j).
 *             When non-NULL the call synchronizes `stream`.
 *   ws        device workspace of ws_bytes >= kq_quantize_layer_workspace(...)
 * Sizes: in % 32 == 0, in % group == 0, in % block == 0, 1 <= out <= 2^22.
 * Synchronizes `stream` before returning (to report KQ_ENOTSPD).
 */
kq_status kq_quantize_layer(const kq_quant_params* p, float* W_rot, const float* HX_rot,
                            const float* HG_rot, int64_t out, int64_t in, uint32_t* packed,
                            float* scales, uint8_t* zeros, uint8_t* codes_opt, double* loss_opt,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * kq_quantize_layer_async -- kq_quantize_layer with its status and losses left in device
 * memory: nothing is waited for, so a caller can quantize many layers in a row, or on
 * several streams at once, and read every status after its own synchronization.
 *
 * Follows: the same passages as kq_quantize_layer, and computes the same results with the
 * same kernels.  Arguments as kq_quantize_layer, except:
 *   loss_dev_opt  device, 2 doubles, or NULL: {direct loss, predicted loss} written when the
 *                 work runs (the workspace must then be sized with losses)
 *   status_dev    device int (required): KQ_OK, or KQ_ENOTSPD when the damped H~_X has a
 *                 non-positive pivot, written when the work runs
 * Argument errors (KQ_EINVAL, KQ_ESHAPE, KQ_ENOTIMPL, KQ_EWORKSPACE) are returned before
 * anything is enqueued; KQ_EHIP if a launch fails.
 */
kq_status kq_quantize_layer_async(const kq_quant_params* p, float* W_rot, const float* HX_rot,
                                  const float* HG_rot, int64_t out, int64_t in, uint32_t* packed,
                                  float* scales, uint8_t* zeros, uint8_t* codes_opt,
                                  double* loss_dev_opt, int* status_dev, void* ws,
                                  size_t ws_bytes, void* stream);

/* Largest workspace kq_quantize_layer_noalloc serves: a layer is accepted when
 * kq_quantize_layer_workspace reports at most this many bytes for it (with losses when
 * losses are requested); e.g. a 2048 x 2048 layer without losses (49 MiB) or a 1024 x 1024
 * layer with them (20.5 MiB). */
#define KQ_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * kq_quantize_layer_noalloc -- kq_quantize_layer with no workspace argument, for callers that
 * cannot allocate device memory at the point of the call (tight serving loops, harnesses
 * that forbid allocation).  Same arguments, steps, outputs and errors as kq_quantize_layer
 * without ws and ws_bytes; it calls no allocating routine.  Its workspace is a fixed array of
 * KQ_NOALLOC_WORKSPACE_BYTES in the library's device memory, one per GPU, held until the
 * process ends; everything in it that must start at zero is cleared by each call.
 *   KQ_EWORKSPACE (before anything is enqueued) when the layer needs more workspace than the
 *   array holds.
 * Calls on one GPU share that GPU's array: calls whose work overlaps on one GPU (different
 * streams, or host threads) race and give undefined results; calls in one stream are
 * ordered.  Synchronizes `stream` before returning, as kq_quantize_layer does.
 */
kq_status kq_quantize_layer_noalloc(const kq_quant_params* p, float* W_rot, const float* HX_rot,
                                    const float* HG_rot, int64_t out, int64_t in,
                                    uint32_t* packed, float* scales, uint8_t* zeros,
                                    uint8_t* codes_opt, double* loss_opt, void* stream);

/*
 * kq_allocate_bits -- per-sublayer bit widths from sensitivities (host only).
 *
 * Follows: KronQ README, opening section and flags table (inter-layer mixed
 * precision, --inter_layer_mp); KronQ arXiv abstract, point 2.  The rule is
 * not stated on the pages; this engine's rule: every sublayer starts at the
 * smallest allowed width; while sum_l bits_l * numel_l stays within
 * floor(sum_l numel_l * target_num / target_den), the sublayer with the
 * largest gain_l = (sens_l * (4^-b_l - 4^-b_next)) / (numel_l * (b_next - b_l))
 * moves to its next allowed width (ties: smallest index).  Deterministic.
 *
 *   sens      host, L fp64 sensitivities (>= 0)
 *   numel     host, L int64 parameter counts (> 0)
 *   allowed   host, n_allowed distinct widths in [1, 16] (any order)
 *   target_num/target_den  average-bit budget as a fraction (> 0)
 *   bits_out  host, L ints
 */
kq_status kq_allocate_bits(const double* sens, const int64_t* numel, int64_t L, const int* allowed,
                           int n_allowed, int64_t target_num, int64_t target_den, int* bits_out);

/*
 * kq_deploy_linear -- one quantized layer applied to an activation vector (batch 1):
 *   y = D_out^-1 P_out^T Qhat P_in D_in^-1 x,   Qhat[r, c] = s[r, g] (q[r, c] - z[r, g]),
 * P = blockdiag(Had_b) diag(S) / sqrt(b) on each side, D = diag(d).
 *
 * Follows: KronQ README, opening section (packed int4/int2 weights dequantized on the fly
 * by a fused dequant + BiIP matvec for single-token decode).  Since kq_biip_rotate gives
 * W~ = P_out D_out W D_in P_in^T and Qhat quantizes W~, y approximates W x.
 *
 *   packed, scales, zeros  device, as written by kq_quantize_layer (natural column order):
 *             uint32 out x (in * bits / 32), fp32 and uint8 out x (in / group)
 *   bits      2 or 4;  group divides in and is a multiple of 128 / bits (or equals in)
 *   d_in, d_out      device fp32 rescale vectors (in, out), or NULL for 1
 *   sign_in, sign_out device int8 +-1 (in, out), or NULL for +1
 *   had_in, had_out  Hadamard blocks: powers of 2 (<= 8192) dividing in / out; 1: none;
 *             0: the largest power of 2 dividing the size, as kq_biip_rotate (KQ_ENOTIMPL
 *             when that exceeds 8192)
 *   x         device fp32 [in];  y  device fp32 [out] (not aliasing x)
 * Sizes: in % 32 == 0; the LDS copy of x~ (in rounded up to 64 * 128 / bits entries, plus
 * 1/16 padding) must fit in 160 KB, i.e. in <= 36864.  No workspace: with had_out > 16 a
 * second kernel on the same stream rotates y in place.  Asynchronous on `stream`;
 * KQ_ESHAPE / KQ_ENOTIMPL / KQ_EINVAL for unsupported arguments, before any launch.
 */
kq_status kq_deploy_linear(const uint32_t* packed, const float* scales, const uint8_t* zeros,
                           int bits, int group, int64_t out, int64_t in, const float* d_in,
                           const float* d_out, const int8_t* sign_in, const int8_t* sign_out,
                           int64_t had_in, int64_t had_out, const float* x, float* y,
                           void* stream);

/*
 * One layer of kq_deploy_linear_group: the arguments of kq_deploy_linear other than in and x
 * (same meaning, layout and limits).
 */
typedef struct kq_deploy_layer {
  const uint32_t* packed;
  const float* scales;
  const uint8_t* zeros;
  int bits;
  int group;
  int64_t out;
  const float* d_in;
  const float* d_out;
  const int8_t* sign_in;
  const int8_t* sign_out;
  int64_t had_in;
  int64_t had_out;
  float* y;
} kq_deploy_layer;

/*
 * kq_deploy_linear_group -- kq_deploy_linear for n_layers (1 .. 8) layers that read the same
 * activation x [in] (a decoder's q/k/v projections, or its gate/up pair), in one launch of
 * the matvec kernel (and at most one of the output rotation).  Each layer has its own codes,
 * width (2 or 4 bits), group, rescale vectors, signs, Hadamard blocks and output y; the
 * outputs must not overlap each other or x.  `layers` is a host array, read during the call.
 * Follows: KronQ README, opening section (the fused dequant + BiIP matvec of the packed
 * deploy path), applied to each layer as kq_deploy_linear.  Errors as kq_deploy_linear,
 * naming the layer; KQ_ESHAPE for n_layers outside 1 .. 8.
 */
kq_status kq_deploy_linear_group(const kq_deploy_layer* layers, int n_layers, int64_t in,
                                 const float* x, void* stream);

/*
 * kq_quantize_two_sided_workspace -- device workspace bytes of kq_quantize_two_sided.
 */
kq_status kq_quantize_two_sided_workspace(const kq_quant_params* p, int64_t out, int64_t in,
                                          size_t* bytes);

/*
 * kq_quantize_two_sided -- two-sided rounding: GPTQ on vec(W) under the Kronecker Hessian
 * H_d = (H_X + lam_X I) (x) (H_G + lam_G I), lam = damp * mean(diag) per factor.
 *
 * Follows: BaKron abstract (two-sided adaptive rounding with a Kronecker-factored Hessian,
 * O(m + n) sequential steps, O(mn(m + n)) work).  With U = U_X (x) U_G (U_* the upper
 * Cholesky factors of the damped inverses) each coordinate W[r, i] is rounded to its grid,
 * e = (w - qhat) / (U_X[i,i] U_G[r,r]), and every W[r', i'] with r' >= r, i' >= i receives
 * -e U_G[r, r'] U_X[i, i'] (the order within that dependency does not change the result).
 * Grids: per (row, group) asymmetric min-max taken from W before rounding (static).  Dead
 * channels (zero diagonal) of either factor zero their column / row of W.
 *
 *   p        bits 2..4, asym 1, act_order 0, w_clip 0, group a multiple of 32 dividing in
 *   W        device fp32, out x in (W~, processed as for kq_quantize_layer), contiguous
 *   HX, HG   device fp32, in x in and out x out symmetric (H~_X, H~_G), contiguous
 *   out, in  multiples of 128 (<= 32768)
 *   packed   device uint32, out x (in * bits / 32): the codes as one bitstream per row
 *   scales   device fp32, out x (in / group);  zeros  device uint8, out x (in / group)
 *   ws       device workspace of kq_quantize_two_sided_workspace bytes
 *   codes_opt device uint8 out x in (the codes unpacked), or NULL
 * Synchronizes `stream` before returning; KQ_ENOTSPD when a damped factor is not positive
 * definite.  KQ_EINVAL / KQ_ESHAPE / KQ_ENOTIMPL / KQ_EWORKSPACE before any launch.
 */
kq_status kq_quantize_two_sided(const kq_quant_params* p, const float* W, const float* HX,
                                const float* HG, int64_t out, int64_t in, uint32_t* packed,
                                float* scales, uint8_t* zeros, void* ws, size_t ws_bytes,
                                uint8_t* codes_opt, void* stream);

/*
 * kq_flipflop_workspace -- device workspace bytes of kq_flipflop for T tokens, n input and m
 * output channels.
 */
kq_status kq_flipflop_workspace(int64_t T, int64_t n, int64_t m, size_t* bytes);

/*
 * kq_flipflop -- the FlipFlop Hessian factors by the alternating fixed-point iteration:
 *   B_0 = I;  for k = 1 .. iters:
 *     A_k = E_t[(g_t^T B_{k-1}^-1 g_t) x_t x_t^T] / m,
 *     B_k = E_t[(x_t^T A_k^-1 x_t) g_t g_t^T] / n,
 * E_t the mean over the T tokens (x_t, g_t: token t's activation and output gradient).
 *
 * Follows: WaterKron and FlipFlop Hessian, Table 1 (row "FlipFlop": input factor
 * E[(g^T B^-1 g) x x^T], output factor E[(x^T A^-1 x) g g^T]) and its caption (alternating
 * fixed-point iteration from the identity).  The 1/m and 1/n are the classical flip-flop's
 * normalization; A (x) B does not depend on it.  Inverses: the reverse Cholesky factor of
 * the current factor without damping (a zero diagonal entry counts as 1); the inverse
 * factor enters the per-token quadratic forms as two bf16 terms (its rounding and the
 * rounding of the remainder, about 16 significant bits) with fp32 accumulation.  Each factor
 * is formed as sum_t a_t s_t^T, the per-token weight applied to one side only: a_t (the
 * weighted token row) as two bf16 terms against the exact bf16 stream s_t, the lower
 * triangle computed and mirrored (exactly symmetric).
 *
 *   X, G     device bf16 bit patterns, T x n and T x m, token-major, leading dims ldx, ldg
 *            (multiples of 8, >= the widths), 16-byte aligned
 *   T        tokens (>= 1);  n, m  channels, multiples of 128 (<= 65536)
 *   iters    1 .. 1000
 *   A, B     device fp32, n x n and m x m, contiguous: A_iters and B_iters (full symmetric)
 *   ws       device workspace of kq_flipflop_workspace(T, n, m) bytes
 *   phase_ms host, 4 doubles, or NULL: HIP-event durations on `stream`, summed over all
 *            half steps, of {factor and inverse factor, per-token quadratic forms,
 *            stream scaling, SYRK}
 * Synchronizes `stream` before returning; KQ_ENOTSPD when a factor has a non-positive
 * pivot (results undefined).  KQ_ESHAPE / KQ_EINVAL / KQ_EWORKSPACE before any launch.
 */
kq_status kq_flipflop(const uint16_t* X, int64_t ldx, const uint16_t* G, int64_t ldg, int64_t T,
                      int64_t n, int64_t m, int iters, float* A, float* B, void* ws,
                      size_t ws_bytes, double* phase_ms, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
