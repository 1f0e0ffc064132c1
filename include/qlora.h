/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA quantized linear layer.
 *
 * The layer keeps a frozen weight W [rows = N = out_features, cols = K =
 * in_features] in NF4 form and adds a trainable low-rank bypass:
 *
 *     y = x W^T + (alpha / r) (x A^T) B^T
 *
 * (26. QLoRA and 4bit Quantization, datawhalechina, Step 3; same formula in
 * 22. QLoRA and 4bit Quantization, Step 4).  W is stored as 4-bit indices into
 * a fixed 16-entry NF4 codebook (26. ..., Step 4 lookup table), one fp32
 * absmax per block of 64 (or 128) consecutive elements of the row-major
 * flattened weight (Gemma lesson 09, sec. 9.2.1: each block is normalised to
 * [-1, 1]; 22. ..., engineering notes: 64 or 128 parameters share one scale),
 * two indices per byte (22. ..., Step 4).  Optionally the block constants are quantised again
 * to 8-bit integers (Gemma lesson 09, sec. 9.2.2 "double quantization";
 * gufacode ch. 4: ~4.5 -> ~4.127 bits per parameter).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers (HIP memory on the current
 *    device) unless a parameter says "host".  Row-major, densely packed.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Every call only enqueues work on that stream and returns; it never
 *    synchronises.  Outputs are valid once the stream reaches the work.
 *  - The caller owns and allocates every buffer, including the workspace.
 *    The library never allocates or frees device memory and keeps no state
 *    between calls apart from read-only kernel code.
 *  - Outputs are overwritten, except dA and dB of the accumulating backward
 *    entry points, which say so.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns a non-zero status and enqueues nothing.  A launch error
 *    reported by the runtime returns QL_EHIP.  No C++ exception crosses the
 *    ABI.  Inputs must be finite; NaN/Inf inputs give unspecified values.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QL_OK 0
#define QL_EINVAL 1       /* null pointer, bad enum value, non-positive size */
#define QL_ESHAPE 2       /* shapes inconsistent or unsupported (e.g. K % 64) */
#define QL_EALIGN 3       /* a pointer lacks the 16-byte alignment required */
#define QL_EUNSUPPORTED 4 /* valid request this build does not implement */
#define QL_EWORKSPACE 5   /* workspace smaller than ql_workspace_bytes() */
#define QL_EHIP 6         /* the HIP runtime reported an error */

/* Element types of activations, weights to quantise, LoRA factors, outputs.
 * The compute dtype of the layer is its activation dtype (Gemma lesson 09,
 * sec. 9.3: the dequantised weight takes the compute dtype, bf16
 * recommended, fp16 where bf16 is unsupported or misbehaves, fp32 possible
 * but costly).  A 16-bit LoRA dtype must equal a 16-bit activation dtype
 * (with fp32 activations it may be QL_BF16). */
#define QL_F32 0
#define QL_BF16 1
#define QL_F16 2 /* IEEE binary16 */

/* Workspace queries (ql_workspace_bytes `op`). */
#define QL_OP_QUANTIZE 0
#define QL_OP_FWD 1
#define QL_OP_BWD 2

/* Format parameters: 64 weights per NF4 block (or 128: 22. QLoRA and 4bit
 * Quantization, engineering notes: 64 or 128 parameters share one scale),
 * 256 block constants per double-quantisation block. */
#define QL_NF4_BLOCK 64
#define QL_NF4_BLOCK_LARGE 128
#define QL_DQ_BLOCK 256

/*
 * An NF4-quantised weight.  n = rows * cols elements, nb = ceil(n / block)
 * block constants, nb2 = ceil(nb / block2) second-level scales.
 *
 *  packed        uint8 [ceil(n/2)]: indices of the row-major flattened weight;
 *                element 2j in bits 7..4 of byte j, element 2j+1 in bits 3..0;
 *                for odd n the last low nibble is 0.
 *  absmax        fp32 [nb]: per-block absolute maximum (double_quant == 0).
 *  absmax_q      int8 [nb]: codes of the centred constants (double_quant == 1).
 *  absmax_scale  fp32 [nb2]: one scale per block2 codes (double_quant == 1).
 *  absmax_mean   fp32 [1]: per-tensor mean of the constants (double_quant == 1).
 *  block is QL_NF4_BLOCK (64) or QL_NF4_BLOCK_LARGE (128); block2 must be
 *  QL_DQ_BLOCK.  The layer entry points need cols % block == 0.
 *
 * Dequantised element i (block b = i / block):
 *   a'  = absmax[b]                                         (no double quant)
 *   a'  = fmaf((float)absmax_q[b], absmax_scale[b / block2], absmax_mean[0])
 *   w^_i = fp32 product codebook[index_i] * a'
 * The struct itself lives in host memory; the pointers it holds are device
 * pointers.  Unused pointers may be NULL.
 */
typedef struct ql_nf4 {
  uint8_t *packed;
  float *absmax;
  int8_t *absmax_q;
  float *absmax_scale;
  float *absmax_mean;
  int64_t rows;
  int64_t cols;
  int32_t block;
  int32_t block2;
  int32_t double_quant;
  int32_t reserved; /* must be 0 */
} ql_nf4;

/*
 * Host only.  Byte sizes of the five buffers of a rows x cols weight:
 * bytes_out[0..4] = packed, absmax, absmax_q, absmax_scale, absmax_mean
 * (entries a format does not use are 0).  Returns QL_OK or QL_EINVAL.
 */
int ql_nf4_sizes(int64_t rows, int64_t cols, int32_t double_quant, size_t bytes_out[5]);

/*
 * Host only.  As ql_nf4_sizes, for blocks of `block` weights (QL_NF4_BLOCK or
 * QL_NF4_BLOCK_LARGE; QL_EINVAL otherwise).  ql_nf4_sizes is this with
 * block = QL_NF4_BLOCK.
 */
int ql_nf4_sizes_block(int64_t rows, int64_t cols, int32_t block, int32_t double_quant,
                       size_t bytes_out[5]);

/*
 * Host only.  Workspace bytes an operation needs (a multiple of 256).
 *   QL_OP_QUANTIZE: M and r ignored, N x K is the weight (double-quant form;
 *                   the single-level form needs none).
 *   QL_OP_FWD / QL_OP_BWD: M tokens, N = out_features, K = in_features, rank r.
 * Returns 0 for invalid sizes.  The forward and backward workspaces never
 * scale with N * K; the quantisation one holds the fp32 block constants
 * (4 bytes per 64 weights) plus a fixed 48 KiB.
 */
size_t ql_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r);

/*
 * NF4-quantise a weight (Gemma lesson 09, sec. 9.2.1 and 9.2.2; 26. ...,
 * Step 2 nearest codepoint).
 *   w         device, q->rows * q->cols elements of w_dtype (QL_F32, QL_BF16 or
 *             QL_F16), 16-byte aligned.
 *   q         host struct describing device outputs: packed and either absmax
 *             (double_quant 0) or absmax_q, absmax_scale, absmax_mean (1).
 * Per block (64 or 128 consecutive elements of the flattened weight):
 * a = max |w|; v = w / a (correctly rounded fp32 division); the
 * index is the nearest codepoint of v, ties to the lower index; a zero block
 * codes every element as index 7 (the exact zero).  Double quantisation:
 * mu = fp32(fp64(S) / nb), where S is the exact sum of all nb constants (an
 * integer multiple of 2^-149 accumulated in integer arithmetic, so exact for
 * any spread of magnitudes), fp64(S) its round-to-nearest-even, and the
 * division correctly rounded;
 * per 256 constants sigma = max|a - mu| / 127 (fp32), code =
 * clamp(round-half-even((a - mu) / sigma), -127, 127), 0 when sigma == 0.
 *   ws, ws_bytes  device workspace of ql_workspace_bytes(QL_OP_QUANTIZE, ...)
 *                 bytes, 256-byte aligned (may be NULL/0 without double quant).
 * Errors: QL_EINVAL, QL_EALIGN, QL_EUNSUPPORTED, QL_EWORKSPACE, QL_EHIP.
 */
int nf4_quantize(const void *w, int32_t w_dtype, const ql_nf4 *q, void *ws, size_t ws_bytes,
                 void *stream);

/*
 * NF4-quantise `count` weights at once (a model's tensors when it is loaded;
 * Gemma lesson 09, sec. 9.2.1 and 9.2.2): the outputs of weight i are those
 * of nf4_quantize(w[i], w_dtype, &q[i], ...), bit for bit, but up to eight
 * weights share one launch (two with double quantisation), so small weights
 * do not each pay a launch.
 *   count     number of weights (0: nothing to do).
 *   w         host array of count device pointers, each q[i].rows *
 *             q[i].cols elements of w_dtype, 16-byte aligned.
 *   q         host array of count structs as for nf4_quantize; all share
 *             block and double_quant.  Outputs of different weights must not
 *             overlap.
 *   ws, ws_bytes  device workspace, 256-byte aligned, of at least the sum
 *             over i of ql_workspace_bytes(QL_OP_QUANTIZE, 0, q[i].rows,
 *             q[i].cols, 0) bytes, weight i using the part after those of
 *             weights 0 .. i-1 (may be NULL/0 without double quant).
 * Every argument is checked before anything is enqueued: on an error no
 * weight has been touched.
 * Errors: QL_EINVAL (count < 0, a NULL array or pointer, mixed block or
 * double_quant, or an invalid struct), QL_EALIGN, QL_EUNSUPPORTED,
 * QL_EWORKSPACE, QL_EHIP.
 */
int nf4_quantize_many(int32_t count, const void *const *w, int32_t w_dtype, const ql_nf4 *q,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * Dequantise a whole NF4 weight to out (device, rows * cols elements of
 * out_dtype: fp32, or bf16 / fp16 as the round-to-nearest-even of the fp32
 * product)
 * (26. ..., Step 4: table[index] * scale; 22. ..., Step 3: restored to a
 * 16-bit float for the matrix product).  out must be 16-byte aligned.
 * Errors: QL_EINVAL, QL_EALIGN, QL_EUNSUPPORTED, QL_EHIP.
 */
int nf4_dequantize(const ql_nf4 *q, void *out, int32_t out_dtype, void *stream);

/*
 * Forward of the layer (26. ..., Step 3):
 *     u = x A^T,   y = x W^^T + s u B^T,   s = fp32(alpha / r)
 * with W^ dequantised on the fly, never stored.
 *   x       device [M, K] act_dtype (QL_BF16 or QL_F16, or QL_F32 for the fp32
 *           path)
 *   W       host struct, rows = N, cols = K, K % W->block == 0
 *   A, B    device [r, K] and [N, r] of lora_dtype (QL_F32, or the 16-bit
 *           activation dtype; QL_BF16 with fp32 activations)
 *   r       1..128;  alpha any finite value
 *   y       device [M, N] act_dtype (overwritten)
 *   u_save  device [M, r] fp32 receiving u, or NULL
 *   ws      device workspace of ql_workspace_bytes(QL_OP_FWD, M, N, K, r)
 * 16-bit activations multiply on the matrix cores in their own format (W^
 * dequantised to it, the rank-r operands rounded to it) with fp32
 * accumulation; fp32 activations compute entirely in fp32.
 * All device pointers 16-byte aligned.
 */
int qlora_linear_fwd(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                     const void *A, const void *B, int32_t lora_dtype, int32_t r, float alpha,
                     void *y, float *u_save, void *ws, size_t ws_bytes, void *stream);

/*
 * The forward of qlora_linear_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): it takes no workspace argument, and neither it nor its
 * kernels allocate.  Its workspace is a fixed array of
 * QL_NOALLOC_WORKSPACE_BYTES bytes inside the library, one per GPU it runs
 * on, held until the process ends; its device address is looked up on the
 * first call on each device.  Arguments and results as qlora_linear_fwd
 * (bit-identical outputs); calls needing more than
 * QL_NOALLOC_WORKSPACE_BYTES of workspace (ql_workspace_bytes(QL_OP_FWD,
 * ...)) return QL_EWORKSPACE and enqueue nothing.  Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (different streams,
 * or host threads) race and give wrong results.  Nothing in the array needs
 * to start at zero (every value is written before it is read).
 * Errors: as qlora_linear_fwd; QL_EWORKSPACE as above; QL_EUNSUPPORTED for
 * a device index of 64 or more.
 */
#define QL_NOALLOC_WORKSPACE_BYTES (32u << 20)
int qlora_linear_fwd_noalloc(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                             const void *A, const void *B, int32_t lora_dtype, int32_t r,
                             float alpha, void *y, float *u_save, void *stream);

/*
 * Forward given the rank-r projection (26. ..., Step 3, with the first
 * bypass product x A^T already at hand, e.g. the u_save of an earlier
 * qlora_linear_fwd on the same x when a forward is recomputed):
 *     y = x W^^T + s u B^T,   s = fp32(alpha / r)
 *   u       device [M, r] fp32, 16-byte aligned
 * Other arguments as for qlora_linear_fwd; no workspace.  With 16-bit
 * activations this is a single matrix-core launch that never splits the
 * contraction.  It is bit-identical to the y of qlora_linear_fwd whenever
 * that call takes the matrix-core GEMM without splitting the contraction
 * either; where it splits (a shape-dependent choice: few output tiles, or
 * tiles that fill the chip better when split) or takes the decode path
 * (M <= 16: the base product and the bypass are summed in fp32 and rounded
 * once, u is formed in its own summation order), the two agree to within
 * 16-bit rounding.
 * Errors: QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EUNSUPPORTED, QL_EHIP.
 */
int qlora_linear_fwd_u(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                       const float *u, const void *B, int32_t lora_dtype, int32_t r,
                       float alpha, void *y, void *stream);

/*
 * Backward of the layer (22. QLoRA and 4bit Quantization, Step 1: the
 * gradient reaches x and the LoRA factors; the frozen base gets none):
 *     u = x A^T (or u_saved),  g = s dy B
 *     dB = s dy^T u   [N, r] fp32
 *     dA = g^T x      [r, K] fp32
 *     dx = dy W^ + g A [M, K] act_dtype   (skipped when dx == NULL)
 * dy [M, N] act_dtype.  Other arguments as for qlora_linear_fwd.  No
 * gradient buffer of size N x K exists anywhere.
 */
int qlora_linear_bwd(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                     const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                     int32_t r, float alpha, const float *u_saved, void *dx, float *dA,
                     float *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * Gradient accumulation (Gemma lesson 9, sec. 9.4.1: several forward and
 * backward passes add their gradients before one optimizer update): as
 * qlora_linear_bwd, but dA and dB receive dA += g^T x and dB += s dy^T u
 * (one fp32 addition per element) instead of being overwritten; dx is still
 * overwritten.  The caller zeroes dA and dB before the first micro-batch.
 */
int qlora_linear_bwd_acc(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                         const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                         int32_t r, float alpha, const float *u_saved, void *dx, float *dA,
                         float *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * LoRA dropout (the pages' training configs set LoraConfig's lora_dropout
 * to 0.05: 26. ..., Step 5.1 and 5.2; 65. QLoRA Selection Project, Step 5.3;
 * Gemma lesson 9, sec. 9.6).  The pages do not say how the mask is drawn.
 * Here it applies to the input of the bypass only (the base product sees x
 * unchanged), with inverted scaling, from a counter-based generator so that
 * the backward regenerates the forward's mask instead of storing it:
 *     xd = d .* x,   d[m][k] = keep[m][k] / (1 - p)   (fp32 of 1 / (1 - p))
 *     keep[m][k] = 1 iff word e % 4 of Philox4x32-10 (Salmon et al., SC'11)
 *                  at counter (e / 4 low 32 bits, e / 4 high 32 bits, 0, 0)
 *                  with key (seed low 32 bits, seed high 32 bits) is
 *                  >= floor(p 2^32) (computed in double),  e = m K + k.
 *   dropout_p  in [0, 1); 0 gives exactly the entry point without dropout.
 *   seed       any 64-bit value; one seed per training step and layer.
 */

/*
 * Forward with LoRA dropout:  u = xd A^T,  y = x W^^T + s u B^T.
 * Arguments as for qlora_linear_fwd (same workspace size).  u_save receives
 * the u of the dropped input, which is what qlora_linear_bwd_dropout's
 * u_saved expects.  Every activation dtype and shape of qlora_linear_fwd.
 * Errors: as qlora_linear_fwd; QL_EINVAL for dropout_p outside [0, 1).
 */
int qlora_linear_fwd_dropout(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                             const void *A, const void *B, int32_t lora_dtype, int32_t r,
                             float alpha, double dropout_p, uint64_t seed, void *y,
                             float *u_save, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward with LoRA dropout (same p and seed as the forward):
 *     u = xd A^T (or u_saved),  g = s dy B,  dB = s dy^T u,
 *     dA = g^T xd,  dx = dy W^ + d .* (g A).
 * accumulate 0 overwrites dA and dB, 1 adds into them (as
 * qlora_linear_bwd_acc).  Workspace as qlora_linear_bwd.  Every activation
 * dtype and shape of qlora_linear_bwd.
 * Errors: as qlora_linear_bwd; QL_EINVAL for dropout_p outside [0, 1) or
 * accumulate not 0/1.
 */
int qlora_linear_bwd_dropout(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                             const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                             int32_t r, float alpha, double dropout_p, uint64_t seed,
                             const float *u_saved, void *dx, float *dA, float *dB,
                             int32_t accumulate, void *ws, size_t ws_bytes, void *stream);

/*
 * The keep mask of the LoRA dropout above as bytes: keep [M, K] uint8 (device,
 * 16-byte aligned) receives 1 for a kept and 0 for a dropped element.  The
 * layer never reads it; it is for callers that want to see the mask.
 * Errors: QL_EINVAL (M or K <= 0, keep NULL, dropout_p outside [0, 1)),
 * QL_EALIGN, QL_EHIP.
 */
int ql_dropout_mask(int64_t M, int64_t K, double dropout_p, uint64_t seed, uint8_t *keep,
                    void *stream);

/*
 * One AdamW step over n fp32 parameters, in place (gufacode fine-tuning
 * chapter 4, "显存计算实战" and "分页优化器": the LoRA factors train with
 * AdamW holding fp32 moments, 8 bytes per parameter; Gemma lesson 9, sec.
 * 9.4: two states per parameter).  The pages do not write the update out;
 * it is the published AdamW definition, every operation one fp32 rounding,
 * none fused, in this order:
 *     p = p * fp32(1 - lr wd)
 *     m = b1 m + (1 - b1) g,   v = b2 v + (1 - b2) (g g)
 *     p = p - step_size * (m / (sqrt(v) / bc2_sqrt + eps))
 * with step_size = fp32(lr / (1 - b1^t)) and bc2_sqrt = fp32(sqrt(1 - b2^t))
 * computed in fp64 from the arguments (t = step >= 1).
 *   param, grad, exp_avg, exp_avg_sq  device fp32 [n], 16-byte aligned
 *   param_bf16  device bf16 [n] receiving the round-to-nearest-even copy of
 *               the new param (what the layer reads as A or B), 8-byte
 *               aligned, or NULL
 * Errors: QL_EINVAL (n < 0, step < 1, a null pointer, b1 or b2 outside
 * [0, 1), eps <= 0, lr or wd NaN), QL_EALIGN, QL_EHIP.  n == 0 enqueues
 * nothing.
 */
int ql_adamw_step(float *param, const float *grad, float *exp_avg, float *exp_avg_sq,
                  uint16_t *param_bf16, int64_t n, double lr, double beta1, double beta2,
                  double eps, double weight_decay, int64_t step, void *stream);

/* Host only: a static string describing a status code. */
const char *ql_strerror(int status);

/* Host only: ABI version (major * 100 + minor).  The minor version grows
 * whenever an entry point is added or a workspace size changes.
 *   106: the decode forward (M <= 16) sizes its workspace for contraction
 *        slices and u slices on every shape.
 *   107: qlora_linear_fwd_noalloc.
 *   108: the double-quantised nf4_quantize keeps 48 KiB of exact partial sums
 *        of the block constants in place of fp64 partials.
 *   109: the decode forward's plan takes longer runs per wave (fewer
 *        contraction slices) on large weights.
 *   110: the LoRA products (u, g, dA, dB) cover several contraction chunks
 *        per workgroup: fewer slices, smaller forward and backward
 *        workspaces on large shapes.
 *   111: the matrix-core input gradient takes N % 8 == 0 and any K of the
 *        layer (before: N % 64 == 0, K % 128 == 0), so more backward
 *        workspaces hold its split-K partials.
 *   112: nf4_quantize_many (several weights per launch).
 *   113: LoRA dropout with fp32 activations, and its backward for every
 *        shape (before: 16-bit activations only, dx with N % 8 == 0). */
int ql_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
