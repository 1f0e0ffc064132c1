// kernels.h -- host-side launchers of the gfx950 kernels (one per .hip file).
// Each launcher enqueues on `stream`, never synchronises, and returns a
// QL_* status.  Shapes and pointers are validated by the C ABI layer before
// a launcher is called.
#pragma once

#include "common.h"

namespace qlora {

// quant.hip
// block: 64 or 128 elements per NF4 block
int launch_nf4_quantize(const void *w, int w_dtype, int64_t n, int block, uint8_t *packed,
                        float *absmax, hipStream_t stream);
// Double-quantised form: quantisation plus exact partial sums of the block
// constants (at most kQdMaxGroups partials of kQdDigits 64-bit counters),
// then mu and the 8-bit codes.  nb >= 2^31 constants: QL_EUNSUPPORTED.
constexpr int kQdMaxGroups = 512;
constexpr int kQdDigits = 12;    // ten 32-bit digit positions, an infinity count, a pad
constexpr int kQdInfDigit = 10;
int launch_nf4_quantize_dq(const void *w, int w_dtype, int64_t n, int block, uint8_t *packed,
                           float *absmax, unsigned long long *partial, int8_t *q, float *sigma,
                           float *mean_out, hipStream_t stream);
// Up to kQmMax weights of one dtype, block size and form in one launch (plus
// one codes launch for the double-quantised form); each weight's outputs
// are those of its own launch above.  partial, q, sigma and mean are read
// only when dq.
constexpr int kQmMax = 8;
int launch_nf4_quantize_many(int count, const void *const *w, int w_dtype, const int64_t *n,
                             int block, bool dq, uint8_t *const *packed, float *const *absmax,
                             unsigned long long *const *partial, int8_t *const *q,
                             float *const *sigma, float *const *mean, hipStream_t stream);
int launch_nf4_dequantize(const uint8_t *packed, int64_t n, BlockScales sc, void *out,
                          int out_dtype, hipStream_t stream);

// lora.hip: the rank-r products around the base matrix product.
//   rows:  out[m][j] = scale * sum_c P[m][c] * Q(j, c)   (u = x A^T, g = s dy B)
//          Q(j, c) = Q[j*ldq_j + c*ldq_c]
//   cols:  out(j, c) = scale * sum_m R[m][j] * P[m][c]    (dA = g^T x, dB = s dy^T u)
size_t lora_rows_partial_floats(int64_t M, int64_t C, int32_t r);
// out may be NULL: then only the partials are produced and the number of
// slices is returned through *slices (the caller reduces them).
int launch_lora_rows_ws(const void *P, int p_dtype, int64_t M, int64_t C, const void *Q,
                        int q_dtype, int64_t ldq_j, int64_t ldq_c, int32_t r, float scale,
                        float *out, float *partial, hipStream_t stream, int *slices = nullptr,
                        const Dropout *drop = nullptr);
size_t lora_cols_partial_floats(int64_t M, int64_t C, int32_t r);
// A fixed-order sum of cols partial slices still to be launched (S == 0:
// none needed): out = scale * sum over S slices, [r][C] or transposed, or
// added into out (accumulate).
struct ColsReduce {
  const float *partial;
  int S;
  int32_t r;
  int64_t C;
  float scale;
  int c_major, accumulate;
  float *out;
};
// accumulate: out += result instead of out = result.  pending: if non-NULL,
// the slice reduction (when one is needed) is not launched but described
// there, for launch_reduce_cols.
int launch_lora_cols(const float *R, int64_t M, int32_t r, const void *P, int p_dtype, int64_t C,
                     float scale, bool out_c_major, float *out, float *partial,
                     hipStream_t stream, bool accumulate = false,
                     const Dropout *drop = nullptr, ColsReduce *pending = nullptr);
// Two such products over the same M tokens and rank r (no dropout), a and b,
// in one launch when both take the matrix-core kernel (else one launch each);
// their slice reductions are described in pending_a / pending_b.
int launch_lora_cols2(const float *Ra, const void *Pa, int64_t Ca, float scale_a, bool cmaj_a,
                      float *out_a, float *partial_a, const float *Rb, const void *Pb, int64_t Cb,
                      float scale_b, bool cmaj_b, float *out_b, float *partial_b, int64_t M,
                      int32_t r, int p_dtype, hipStream_t stream, bool accumulate,
                      ColsReduce *pending_a, ColsReduce *pending_b);
// one launch for up to two pending reductions (empty ones are skipped)
int launch_reduce_cols(const ColsReduce &a, const ColsReduce &b, hipStream_t stream);

// simple.hip: fp32-accumulating tiled kernels for any activation dtype.
int launch_simple_fwd(const void *x, int act_dtype, int64_t M, const uint8_t *packed,
                      BlockScales sc, int64_t N, int64_t K, const float *u, const void *B,
                      int lora_dtype, int32_t r, float s, void *y, hipStream_t stream);
int launch_simple_dx(const void *dy, int act_dtype, int64_t M, const uint8_t *packed,
                     BlockScales sc, int64_t N, int64_t K, const float *g, const void *A,
                     int lora_dtype, int32_t r, void *dx, hipStream_t stream,
                     const Dropout *drop = nullptr, float dscale = 1.0f);

// gemv.hip: decode-sized forward (M <= 16, 16-bit activations): computes
// u = x A^T itself and writes it to u_save when non-null.  One launch, or,
// when part is non-null and the weight has few row groups and several
// rounds of 4096 columns, the contraction split over workgroups with fp32
// partials in part (gemv_fwd_partial_floats floats) and a second launch
// that sums them.
size_t gemv_fwd_partial_floats(int64_t M, int64_t N, int64_t K, int32_t r);
// y[m][n] = RN(fmaf(s, sum_j u_j B_nj, sum of S slices of part [S][M][N])),
// u = uscale * (sum of U slices of upart [U][M][r]) (stored to u_save when
// non-null; uscale = 1 / (1 - p) under LoRA dropout, else 1).
int launch_fwd_finish(int act_dtype, int lora_dtype, const float *part, int S,
                      const float *upart, int U, int64_t M, int64_t N, int32_t r, const void *B,
                      float s, void *y, float *u_save, hipStream_t stream, float uscale = 1.0f);
// drop: LoRA dropout of the bypass input (NULL for none), dscale = 1 / (1 - p).
int launch_gemv_fwd(const void *x, int act_dtype, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                    int lora_dtype, int32_t r, float s, void *y, float *u_save,
                    hipStream_t stream, float *part, const Dropout *drop = nullptr,
                    float dscale = 1.0f);

// gemm.hip: matrix-core forward and input-gradient products for 16-bit
// activations (act_dtype QL_BF16 or QL_F16; a 16-bit lora_dtype equals it).
// part: fp32 workspace of gemm_*_partial_floats floats for split-K
// launches, or NULL (no split).
// tiny.hip: fp32 activations at small sizes (M <= 16, r <= 64, M N K <=
// 2^22): each pass of the layer in one workgroup, no workspace.
bool tiny_preferred(int act_dtype, int64_t M, int64_t N, int64_t K, int32_t r);
int launch_tiny_fwd(const void *x, int64_t M, const uint8_t *packed, BlockScales sc, int64_t N,
                    int64_t K, const void *A, const void *B, int lora_dtype, int32_t r, float s,
                    void *y, float *u_save, hipStream_t stream);
int launch_tiny_bwd(const void *dy, const void *x, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                    int lora_dtype, int32_t r, float s, const float *u_saved, void *dx, float *dA,
                    float *dB, bool accumulate, hipStream_t stream);
size_t gemm_fwd_partial_floats(int64_t M, int64_t N, int64_t K);
// Few-token forward (17..128 tokens, 16-bit activations) in two launches: the
// 64-token GEMM tiles plus u slice workgroups, then the slice sum with the
// bypass (part: gemm_fwd_fused_partial_floats floats); drop as for the
// decode forward.
bool gemm_fwd_fused_preferred(int64_t M);
size_t gemm_fwd_fused_partial_floats(int64_t M, int64_t N, int64_t K, int32_t r);
int launch_gemm_fwd_fused(const void *x, int act_dtype, int64_t M, const uint8_t *packed,
                          BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                          int lora_dtype, int32_t r, float s, void *y, float *u_save,
                          hipStream_t stream, float *part, const Dropout *drop = nullptr,
                          float dscale = 1.0f);
size_t gemm_dx_partial_floats(int64_t M, int64_t N, int64_t K);
int launch_gemm_fwd(const void *x, int act_dtype, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const float *u, const void *B,
                    int lora_dtype, int32_t r, float s, void *y, hipStream_t stream, float *part);
bool gemm_dx_supported(int64_t N, int64_t K);
int launch_gemm_dx(const void *dy, int act_dtype, int64_t M, const uint8_t *packed,
                   BlockScales sc, int64_t N, int64_t K, const float *g, const void *A,
                   int lora_dtype, int32_t r, void *dx, hipStream_t stream, float *part,
                   const Dropout *drop = nullptr, float drop_scale = 1.0f);
// dropout.hip: the keep mask of the LoRA dropout as bytes (0/1), [M, K]
int launch_dropout_mask(int64_t M, int64_t K, const Dropout &d, uint8_t *keep,
                        hipStream_t stream);

// optim.hip: one AdamW step (scalars from the fp64 hyperparameters)
int launch_adamw(float *p, const float *g, float *m, float *v, uint16_t *p_bf16, int64_t n,
                 double lr, double beta1, double beta2, double eps, double weight_decay,
                 int64_t step, hipStream_t stream);

}  // namespace qlora
