/*
 * sbl.h -- C ABI of the Sparse-BitLinear forward library for AMD MI355X (gfx950).
 *
 * The library computes the forward pass of a Sparse-BitLinear layer as the
 * Sparse-BitNet summary (paper-graph-ui, section 3.4 "Detailed, Sentence-Based
 * Technical Breakdown") states it:
 *   x~    = Q_a(x)                      per-token absmax int8 activations
 *   M     = Pi_{N:M}(|W|)               keep-mask from master-weight magnitudes
 *   W_q   = RoundClip(W/(gamma+eps),-1,1), gamma = mean |W| over the tensor
 *   W_eff = W_q (.) M                   quantize, then apply the mask
 *   y     = s * (W_eff x~)              int32 accumulation, one fp rescale
 *
 * Conventions shared by every call
 *   - Every device pointer is caller-owned; the library never allocates,
 *     frees or retains memory. Pointers must be 16-byte aligned.
 *   - Calls only enqueue work on `stream` and return; nothing waits for the
 *     device. Scalars computed on the device (gamma, sw) stay there.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     failure the first error is returned and no work is enqueued. Launch
 *     failures are reported as SBL_ERR_HIP. No exception crosses the ABI.
 *   - Matrices are row-major: x [T, K] (row stride ldx elements), W [O, K],
 *     y [T, O]. N:M groups run along K inside each row of W, starting at k=0.
 *   - Supported: M in {4, 8}, 1 <= N <= M, K % M == 0, 1 <= K <= 2^24.
 *     T = 0 (or O = 0 where noted) is a valid empty call that enqueues nothing.
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *   - Thread safety: calls are stateless apart from a per-device property cache.
 *
 * Packed ternary-plus-index weight format (this library's own layout; the
 * pages only fix that four ternary values fit one byte -- BitNet b1.58 2B4T
 * summary, section 3.4 "Inference Implementation: GPU" -- and that the
 * structured-sparse kernels share one weight layout -- Sparse-BitNet
 * paperlayer.ai summary, appendix A.2):
 *   2-bit code: 0 -> 00, +1 -> 01, -1 -> 11.
 *   Byte-sliced word: a uint32 holding 16 two-bit fields, field u at bit
 *     8*(u%4) + 2*(u/4); (word >> 2j) & 0x03030303 yields fields 4j..4j+3 one
 *     per byte, so one byte-permute turns them into four int8 values.
 *   Each row of W is one record of fixed pitch (sbl_packed_bytes / O), so
 *   packed buffers of several tensors with the same K concatenate along O.
 *   INDEX FORM (N=2 with M=4 or M=8; feeds the gfx950 2:4 sparse MFMA
 *     directly -- every 2:8 pattern is also a 2:4 pattern):
 *     pitch = ceil(K/128)*32 bytes (+ ceil(K/128)*16 for M=8). Chunk c (k in
 *     [32c, 32c+32), 8 groups q of 4) is two little-endian uint32: word 0
 *     holds, as byte-sliced field v = 2q + j, the code of the j-th selected
 *     slot (ascending) of group q; word 1 holds the selected slot indices:
 *     bits [4q+1:4q] first, [4q+3:4q+2] second. The selected slots are the
 *     kept ones; for 2:8 a group of 4 holding fewer than two kept slots is
 *     completed with its lowest free slots (code 0), and ceil(K/128)*4 mask
 *     words follow the chunks (bit j of word c = mask[32c + j]). Groups past
 *     K: slots (0,1), codes 0. 2 bits per weight (2:8: 3).
 *   DENSE FORM (every other N:M):
 *     pitch = ceil(K/64)*16 + ceil(K/128)*16 bytes. First ceil(K/64)*4 uint32
 *     byte-sliced words of W_eff codes (word c: k = 16c + u as field u), then
 *     ceil(K/128)*4 uint32 mask words (bit j of word c = mask[32c + j]).
 *     Everything past K is zero. 3 bits per weight (2 read by the GEMM).
 */
#ifndef SBL_H
#define SBL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SBL_OK = 0,
  SBL_ERR_NULL = 1,       /* a required pointer is NULL */
  SBL_ERR_SHAPE = 2,      /* a size is negative/zero where not allowed, K % M != 0, too large, ldx < K */
  SBL_ERR_NM = 3,         /* M not in {4,8} or N not in [1, M] */
  SBL_ERR_DTYPE = 4,      /* dtype not SBL_BF16 / SBL_FP32 */
  SBL_ERR_ALIGN = 5,      /* a device pointer is not 16-byte aligned */
  SBL_ERR_WORKSPACE = 6,  /* workspace too small (or NULL while bytes are needed) */
  SBL_ERR_HIP = 7,        /* a HIP runtime call or kernel launch failed */
  SBL_ERR_VALUE = 8       /* eps not a positive, normal, finite float */
} sbl_status;

typedef enum { SBL_BF16 = 0, SBL_FP32 = 1 } sbl_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char* sbl_status_string(int status);

/* Library version string, e.g. "sbl 0.1 gfx950". */
const char* sbl_version(void);

/*
 * a1. Per-token absmax int8 activation quantization.
 * Sparse-BitNet summary, section 3.4 "Activation quantization" (Clip(x *
 * 127/(max|x| + eps), -128, 127)); BitNet b1.58 2B4T summary, section 3.4
 * "Activation Quantization: Per-Token Absmax" (one scale per token, nearest
 * integer). For each row t of x, in IEEE fp32:
 *   m = max_k |x[t,k]|, d = m + eps_a, s = 127 / d,
 *   xq[t,k] = clamp(rint_half_even(x[t,k] * s), -128, 127), sx[t] = d / 127.
 * x: device, [T, K] of xdt with row stride ldx >= K elements.
 * xq: device int8 [T, K] contiguous (written). sx: device float [T] (written).
 */
sbl_status sbl_quant_act(const void* x, sbl_dtype xdt, int64_t T, int64_t K, int64_t ldx,
                         float eps_a, int8_t* xq, float* sx, hipStream_t stream);

/*
 * a1 with the normalization before it fused in: x~ = Q_a(RMSNorm(x)).
 * Sparse-BitNet summary, section 3.4 (Algorithm 1 walk-through: the
 * activations are normalized -- RMSNorm in BitNet -- then quantized); BitNet
 * b1.58 2B4T summary, section 3.2 (subln normalization, no bias terms).
 * The pages fix no arithmetic for the norm; per row t this call computes
 *   sq_k = fp32(x_k * x_k), S = their exact sum rounded once to the nearest
 *     fp64 (independent of the order of the terms),
 *   r = fp32(1 / sqrt(S / K + eps_n)) in fp64,
 *   z_k = fp32(fp32(x_k * r) * gain[k])  (gain NULL: z_k = fp32(x_k * r)),
 * and then exactly sbl_quant_act on z (xq and sx as there; sx refers to z).
 * gain: optional device float [K] (16-byte aligned). eps_n > 0, normal.
 * Rows must be 16-byte aligned (ldx * element size % 16 == 0) and K a
 * multiple of 8 (bf16) or 4 (fp32), else SBL_ERR_SHAPE. |x| < 2^64 (finite
 * squares), else the result is unspecified.
 */
sbl_status sbl_rmsnorm_quant_act(const void* x, sbl_dtype xdt, const float* gain, int64_t T,
                                 int64_t K, int64_t ldx, float eps_n, float eps_a, int8_t* xq,
                                 float* sx, hipStream_t stream);

/* Workspace bytes sbl_quant_mask_weight needs for an [O, K] tensor. */
sbl_status sbl_quant_mask_weight_workspace(int64_t O, int64_t K, size_t* bytes);

/*
 * a2 + a3 + a4. Absmean scale, N:M mask, RoundClip and mask application,
 * packing -- the weight side of the forward, with the mask recomputed on
 * every call. Sparse-BitNet summary, section 3.4: "Step 1: Compute the
 * Rescaling Factor", "Step 2: Rescale and RoundClip" (Eq. 1), "N:M Mask
 * Generation", "Composition Order: Quant-Then-Mask".
 *   gamma = fp32( RN64(sum |W|) / (O*K) ), the sum exact and order-free;
 *   sw = fp32(gamma + eps_w);
 *   mask: per row and group of M along K keep the N largest |W| (ties: lower
 *         index first; exactly N kept);
 *   code = clamp(rint_half_even(fp32(W / sw)), -1, 1); W_eff = code * mask.
 * w: device [O, K] master weights of wdt (fp32 or bf16), contiguous.
 * w_eff (int8 [O,K]), mask (uint8 0/1 [O,K]), packed (sbl_packed_bytes bytes),
 *   sw_rows (float [O], every entry = sw): optional outputs, may be NULL.
 * gamma_sw: device float[2] (required) <- {gamma, sw}.
 * ws: device workspace of at least sbl_quant_mask_weight_workspace bytes;
 *   its contents need no initialisation and are scratch after the call.
 * O * K must be in [1, 2^31).
 */
sbl_status sbl_quant_mask_weight(const void* w, sbl_dtype wdt, int64_t O, int64_t K, int N, int M,
                                 float eps_w, int8_t* w_eff, uint8_t* mask, void* packed,
                                 float* gamma_sw, float* sw_rows, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * sbl_quant_mask_weight without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Arguments, validation, kernels and
 * results are those of sbl_quant_mask_weight; the workspace is a fixed
 * 64 KiB array in device memory that the library holds on every GPU it runs
 * on until the process ends (the call needs 40 KiB for any shape, so no
 * size is refused for want of scratch; SBL_ERR_WORKSPACE would report it).
 * The call allocates and frees nothing. Its first call on a device looks up
 * that device's copy of the array (SBL_ERR_HIP if the lookup fails).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on different streams, or from several host threads onto
 * streams that run concurrently) race and give undefined results; calls
 * ordered on one stream are safe. The array's contents need no clearing:
 * every byte the kernels read there was written earlier in the same call.
 */
sbl_status sbl_quant_mask_weight_noalloc(const void* w, sbl_dtype wdt, int64_t O, int64_t K,
                                         int N, int M, float eps_w, int8_t* w_eff,
                                         uint8_t* mask, void* packed, float* gamma_sw,
                                         float* sw_rows, hipStream_t stream);

/*
 * One weight tensor of sbl_quant_mask_weight_batch. Every pointer is a
 * device pointer with the meaning, layout and optionality of the argument of
 * the same name of sbl_quant_mask_weight; O and K likewise.
 */
typedef struct sbl_weight_prep {
  const void* w;
  int64_t O;
  int64_t K;
  int8_t* w_eff;
  uint8_t* mask;
  void* packed;
  float* gamma_sw;
  float* sw_rows;
  /* Mask diagnostics, all optional (NULL = not computed). Sparse-BitNet
   * summary, section 3.4 / 5: the mask flip rate r_t (Eq. 6: the mask
   * positions that change between consecutive steps) and the per-block
   * pruning threshold of the magnitude-stratification analysis (Fig. 6: the
   * magnitude of the (N+1)-th largest weight of each group).
   * mask_bits: device uint32 [O][C], C = ceil(K/128)*4 words per row; bit e of
   *   word (o, c) is the keep bit of k = 32c + e (0 for k >= K) -- the layout
   *   of the dense-form mask area.
   * prev_mask_bits: device, same layout (e.g. the previous step's mask_bits);
   *   given together with flips and mask_bits.
   * flips: device uint64, set to the number of positions whose keep bit differs
   *   from prev_mask_bits (r_t = flips / (O*K)); counted by one more small
   *   kernel after the mask pass.
   * group_thr: device float [O][K/M]: (N+1)-th largest |w| of each group of M
   *   along K (the largest dropped magnitude; 0 when N == M). */
  uint32_t* mask_bits;
  const uint32_t* prev_mask_bits;
  unsigned long long* flips;
  float* group_thr;
  /* Which recipe (Sparse-BitNet summary, section 3.4 "Where the mask is
   * computed" and the Figure 3a ablations): SBL_PREP_METHOD (0) ranks the mask
   * on the master magnitudes |W| -- the method; SBL_PREP_MASK_FROM_TERNARY (1)
   * ranks it on the ternary magnitudes |W_q| (ties: lower index first), the
   * ablated variant; gamma covers all of W in both. SBL_PREP_MASK_THEN_QUANT
   * (2), the composition-order ablation (section 3.4 "Composition Order"),
   * keeps the master-ranked mask but takes gamma over the kept weights only:
   * gamma = fp32(RN_fp64(sum of kept |w|) / (O * K/M * N)); a batch is either
   * all of variant 2 or has none. group_thr is the largest dropped |w| of each
   * group under the mask actually used. */
  int32_t variant;
} sbl_weight_prep;

#define SBL_PREP_METHOD 0
#define SBL_PREP_MASK_FROM_TERNARY 1
#define SBL_PREP_MASK_THEN_QUANT 2

#define SBL_MAX_PREP_BATCH 8

/* Workspace bytes sbl_quant_mask_weight_batch needs for count tensors. */
sbl_status sbl_quant_mask_weight_batch_workspace(int count, size_t* bytes);

/*
 * a2 + a3 + a4 for count (1..SBL_MAX_PREP_BATCH) independent weight tensors
 * of one dtype and one N:M pattern -- e.g. all projections of a layer -- in
 * three kernel launches in total instead of three per tensor. The same
 * passages of the Sparse-BitNet summary apply per tensor; each tensor gets
 * exactly the outputs sbl_quant_mask_weight gives it (its own gamma and sw,
 * mask, codes, packing).
 * items: host array of count descriptors, read during the call only.
 * Tensors may have different O and K; no output may overlap another
 * tensor's input or output.
 * ws: device workspace of at least sbl_quant_mask_weight_batch_workspace
 *   bytes; no initialisation needed, scratch after the call.
 * Errors: as sbl_quant_mask_weight, checked for every item before anything
 * is enqueued; count out of range -> SBL_ERR_SHAPE; prev_mask_bits, flips
 * and mask_bits not all given when either of the first two is -> SBL_ERR_NULL;
 * an unknown variant, or variant 2 mixed with others in one batch ->
 * SBL_ERR_VALUE.
 */
sbl_status sbl_quant_mask_weight_batch(const sbl_weight_prep* items, int count, sbl_dtype wdt,
                                       int N, int M, float eps_w, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Size in bytes of the packed format for an [O, K] N:M tensor (O * pitch). */
sbl_status sbl_packed_bytes(int64_t O, int64_t K, int N, int M, size_t* bytes);

/*
 * Pack / unpack between (W_eff, mask) and the packed format above.
 * w_eff: device int8 [O,K] in {-1,0,1}, zero wherever mask is 0; mask: device
 * uint8 [O,K] with exactly N ones per group of M. Other contents give an
 * unspecified (but in-bounds) packed result. unpack(pack(w, m)) == (w, m).
 */
sbl_status sbl_pack(const int8_t* w_eff, const uint8_t* mask, int64_t O, int64_t K, int N, int M,
                    void* packed, hipStream_t stream);
sbl_status sbl_unpack(const void* packed, int64_t O, int64_t K, int N, int M, int8_t* w_eff,
                      uint8_t* mask, hipStream_t stream);

/*
 * a5 + a6. int8 x ternary N:M GEMM with an int32 accumulator, dequantized.
 * Sparse-BitNet summary, section 3.4 "The Full Sparse-BitLinear Layer"
 * (y = s * (W_eff x~), one scalar absorbs both scales; Eq. 4).
 *   acc[t,o] = sum_k xq[t,k] * W_eff[o,k]          (exact int32)
 *   y[t,o]   = fp32(fp32(float(acc) * sx[t]) * sw[o * sw_inc]) -> ydt (bf16: RNE)
 * xq: device int8 [T,K]; sx: device float [T]; packed: device, packed format;
 * sw: device float, one value per row of W (sw_inc = 1) or one for all rows
 *   (sw_inc = 0), e.g. &gamma_sw[1] from sbl_quant_mask_weight;
 * y: device [T,O] of ydt (written); acc: optional device int32 [T,O].
 * 2:4 weights run on the gfx950 sparse MFMA (smfmac); other N:M on dense
 * int8 MFMA; small T uses a bandwidth-oriented variant. Same results.
 * T = 0 or O = 0: nothing is enqueued. Extent limits (SBL_ERR_SHAPE beyond,
 * checked before anything else is looked at): T < 2^31, O < 2^31, and each
 * operand below 2^31 -- T*K (xq bytes), O*pitch (packed bytes), T*O (y and
 * acc elements); the kernels address them with 32-bit offsets.
 */
sbl_status sbl_gemm(const int8_t* xq, const float* sx, const void* packed, const float* sw,
                    int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N, int M, void* y,
                    sbl_dtype ydt, int32_t* acc, hipStream_t stream);

/* Workspace bytes for sbl_linear_fwd (prepacked != 0: weights come packed). */
sbl_status sbl_linear_fwd_workspace(int64_t T, int64_t O, int64_t K, int N, int M, int prepacked,
                                    size_t* bytes);

/*
 * The whole forward: a1 on x, then either a2-a4 on w_master (mask recomputed
 * this call) or the caller's prepacked weights with their sw, then a5 + a6.
 * Sparse-BitNet summary, section 3.4 "The Full Sparse-BitLinear Layer"
 * (Algorithm 1 forward, Algorithm 2).
 * x: device [T,K] of xdt, contiguous. Exactly one of w_master (device [O,K]
 * of wdt) and prepacked (device packed buffer, with sw_prepacked / sw_inc as
 * in sbl_gemm) must be non-NULL. y: device [T,O] of ydt.
 * ws: at least sbl_linear_fwd_workspace bytes (scratch).
 * Extent limits as sbl_gemm (SBL_ERR_SHAPE beyond).
 */
sbl_status sbl_linear_fwd(const void* x, sbl_dtype xdt, const void* w_master, sbl_dtype wdt,
                          const void* prepacked, const float* sw_prepacked, int64_t sw_inc,
                          int64_t T, int64_t O, int64_t K, int N, int M, float eps_a, float eps_w,
                          void* y, sbl_dtype ydt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of the layer under the Dual straight-through estimator
 * (Sparse-BitNet summary, section 3.4 "Gradient Estimation: The Dual
 * Straight-Through Estimator" and the backward steps of the Algorithm 1
 * walk-through; Algorithm 2's WeightQuantMasked hands its output gradient
 * back unchanged). The forward is y = x~ W~^T with x~ = sx * xq (the
 * dequantized activation) and W~ = sw * W_eff, so
 *   dX = dY W~      -- the gradient at x~, which the STE of Q_a passes to x;
 *   dW = dY^T x~    -- the gradient at W~, which the Dual STE passes to every
 *                      master weight, kept or pruned, with no clip window.
 * Both contractions run on the bf16 matrix cores with fp32 accumulation; dY
 * is bf16 (the training dtype of the pages) and x~ enters dW as bf16 (see
 * sbl_act_dequant). Shapes: O % 8 == 0 and K % 8 == 0 (16-byte vectors along
 * both), plus the conventions above; ldy >= O with ldy % 8 == 0.
 */

/*
 * x~ as the weight gradient consumes it: xt[t,k] = bf16 of fp32(xq[t,k]) *
 * sx[t], rounded to nearest even. xq: device int8 [T,K] and sx: device
 * float[T] from sbl_quant_act; xt: device bf16 [T,K]. K % 8 == 0 or
 * SBL_ERR_SHAPE; T = 0 enqueues nothing.
 */
sbl_status sbl_act_dequant(const int8_t* xq, const float* sx, int64_t T, int64_t K, void* xt,
                           hipStream_t stream);

/*
 * dX[t,k] (+)= sum_o dY[t,o] * sw_o * W_eff[o,k].
 * dy: device bf16 [T, ldy], columns 0..O-1 used. packed, sw_rows: the
 * forward's packed weights ([O] concatenated rows, N:M as packed) and their
 * per-row sw (sbl_gemm's sw with sw_inc = 1). The O rows form nseg (1..4)
 * segments of seg_rows[i] rows each (seg_rows may be NULL when nseg = 1:
 * one segment of O rows); sw must be constant within a segment (one weight
 * tensor each) and is read from its first row. Each segment's sum is scaled
 * by its sw in fp32 and the segments added in order.
 * dx: device [T, lddx] of dxdt (lddx >= K); accumulate != 0 adds to what dx
 * holds (for bf16: one rounding of fp32(dx) + result), else overwrites.
 * Errors: seg_rows not summing to O, a segment empty or not a multiple of 8,
 * nseg out of range -> SBL_ERR_SHAPE. T = 0 enqueues nothing.
 */
sbl_status sbl_linear_bwd_dx(const void* dy, int64_t ldy, const void* packed, const float* sw_rows,
                             int64_t T, int64_t O, int64_t K, int N, int M, const int64_t* seg_rows,
                             int nseg, void* dx, sbl_dtype dxdt, int64_t lddx, int accumulate,
                             hipStream_t stream);

/*
 * dW[o,k] = sum_t dY[t,o] * xt[t,k]: the master-weight gradient of every
 * weight, pruned ones included (the Dual STE).
 * dy: device bf16 [T, ldy]; xt: device bf16 [T,K] from sbl_act_dequant;
 * dw: device [O,K] of dwdt, overwritten (T = 0 writes zeros; dy and xt may
 * then be NULL).
 * keep_bits: NULL for the method. Non-NULL selects the gated estimator the
 * pages ablate against it (section 3.4 "Gradient Estimation", the
 * mask-gated gradients of prior sparse training, "mask without grad" in
 * Figure 3): dW = M (.) dY^T x~, zero wherever the mask prunes. Layout as
 * sbl_weight_prep.mask_bits: device uint32 [O][ceil(K/128)*4], bit e of word
 * c of row o = M[o, 32c + e].
 */
sbl_status sbl_linear_bwd_dw(const void* dy, int64_t ldy, const void* xt, int64_t T, int64_t O,
                             int64_t K, const uint32_t* keep_bits, void* dw, sbl_dtype dwdt,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SBL_H */
