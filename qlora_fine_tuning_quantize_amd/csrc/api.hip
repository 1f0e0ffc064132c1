// api.hip -- the C ABI declared in include/qlora.h: argument checks on the
// host, workspace carve-up, and the choice of kernels.  No allocation, no
// synchronisation, no state.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kernels.h"

using namespace qlora;

// Workspace of qlora_linear_fwd_noalloc: a fixed device array (one copy per
// GPU, held until the process ends).  Host code never passes its name to a
// kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and that
// address is used instead.
static __device__ __align__(256) uint8_t scratch[QL_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_dtype(int32_t d) {
  return (d == QL_F32 || d == QL_BF16 || d == QL_F16) ? QL_OK : QL_EINVAL;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validates the quantised-weight descriptor (pointers it must hold for its
// format, fixed block sizes, alignment of the packed array).
int check_nf4(const ql_nf4 *q) {
  if (!q) return QL_EINVAL;
  if (q->rows <= 0 || q->cols <= 0) return QL_EINVAL;
  if (q->double_quant != 0 && q->double_quant != 1) return QL_EINVAL;
  if (q->reserved != 0) return QL_EINVAL;
  if ((q->block != QL_NF4_BLOCK && q->block != QL_NF4_BLOCK_LARGE) || q->block2 != QL_DQ_BLOCK)
    return QL_EUNSUPPORTED;
  if (!q->packed) return QL_EINVAL;
  if (q->double_quant) {
    if (!q->absmax_q || !q->absmax_scale || !q->absmax_mean) return QL_EINVAL;
  } else if (!q->absmax) {
    return QL_EINVAL;
  }
  if (!aligned16(q->packed)) return QL_EALIGN;
  return QL_OK;
}

BlockScales scales_of(const ql_nf4 *q) {
  BlockScales sc;
  sc.absmax = q->double_quant ? nullptr : q->absmax;
  sc.q = q->absmax_q;
  sc.sigma = q->absmax_scale;
  sc.mu = q->absmax_mean;
  sc.shift = q->block == 128 ? 1 : 0;
  return sc;
}

// Workspace layouts (offsets are multiples of 256 bytes).
struct QuantWs {
  size_t absmax, partial, total;
};
QuantWs quant_ws(int64_t n) {
  const int64_t nb = ceil_div(n, QL_NF4_BLOCK);
  QuantWs w;
  w.absmax = 0;
  w.partial = round_up((size_t)nb * 4);
  w.total = w.partial + round_up((size_t)kQdMaxGroups * kQdDigits * 8);
  return w;
}

// The split-K partial tiles of a GEMM start at `rows`: the LoRA partials
// stored there are dead once the GEMM (issued later on the same stream) runs.
// Token counts up to 16 take the decode forward (a weight-streaming launch
// that also computes u in a few workgroups of its own, then a launch that
// sums the contraction slices and adds the bypass); larger ones the
// matrix-core GEMMs.
bool gemv_fwd_preferred(int64_t M, int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return M <= 16;
}

struct FwdWs {
  size_t u, rows, total;
};
FwdWs fwd_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  FwdWs w;
  w.u = 0;
  w.rows = round_up((size_t)M * r * 4);
  w.total = w.rows + round_up(lora_rows_partial_floats(M, K, r) * 4);
  const size_t gemm_end = w.rows + round_up(gemm_fwd_partial_floats(M, N, K) * 4);
  if (gemm_end > w.total) w.total = gemm_end;
  if (M <= 16) {  // a decode forward's split partials, in the same region
    const size_t gemv_end = w.rows + round_up(gemv_fwd_partial_floats(M, N, K, r) * 4);
    if (gemv_end > w.total) w.total = gemv_end;
  }
  // a few-token forward's slice partials of y and u, in the same region
  const size_t fused_end = w.rows + round_up(gemm_fwd_fused_partial_floats(M, N, K, r) * 4);
  if (fused_end > w.total) w.total = fused_end;
  return w;
}

// dB's and dA's slice partials have regions of their own (cols, cols2): their
// two reductions run as one launch after both products.
struct BwdWs {
  size_t u, g, rows, cols, cols2, total;
};
BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdWs w;
  w.u = 0;
  w.g = round_up((size_t)M * r * 4);
  w.rows = w.g + round_up((size_t)M * r * 4);
  size_t rows_f = lora_rows_partial_floats(M, K, r);
  size_t rows_f2 = lora_rows_partial_floats(M, N, r);
  if (rows_f2 > rows_f) rows_f = rows_f2;
  w.cols = w.rows + round_up(rows_f * 4);
  w.cols2 = w.cols + round_up(lora_cols_partial_floats(M, N, r) * 4);
  w.total = w.cols2 + round_up(lora_cols_partial_floats(M, K, r) * 4);
  if (gemm_dx_supported(N, K)) {
    const size_t gemm_end = w.rows + round_up(gemm_dx_partial_floats(M, N, K) * 4);
    if (gemm_end > w.total) w.total = gemm_end;
  }
  return w;
}

int check_linear_common(int32_t act_dtype, int64_t M, const ql_nf4 *W, const void *A,
                        const void *B, int32_t lora_dtype, int32_t r, float alpha) {
  int st = check_nf4(W);
  if (st) return st;
  if (check_dtype(act_dtype) || check_dtype(lora_dtype)) return QL_EINVAL;
  // 16-bit activations: the LoRA factors are fp32 or of the same format
  if (act_dtype != QL_F32 && lora_dtype != QL_F32 && lora_dtype != act_dtype)
    return QL_EUNSUPPORTED;
  if (M <= 0 || r <= 0) return QL_EINVAL;
  if (r > 128) return QL_EUNSUPPORTED;
  if (W->cols % W->block != 0) return QL_ESHAPE;  // blocks never straddle weight rows
  if (!A || !B) return QL_EINVAL;
  if (!aligned16(A) || !aligned16(B)) return QL_EALIGN;
  if (!(alpha == alpha) || alpha - alpha != 0.0f) return QL_EINVAL;  // not finite
  return QL_OK;
}

// LoRA dropout parameters of a call: keep threshold floor(p 2^32) on the
// 32-bit draw (computed in double), inverted scale fp32(1 / (1 - p)), key =
// the 64-bit seed.  p must lie in [0, 1).
int dropout_of(double p, uint64_t seed, Dropout &d, float &scale) {
  if (!(p >= 0.0 && p < 1.0)) return QL_EINVAL;
  d.k0 = (uint32_t)seed;
  d.k1 = (uint32_t)(seed >> 32);
  d.thr = (uint32_t)floor(p * 4294967296.0);
  scale = (float)(1.0 / (1.0 - p));
  return QL_OK;
}

}  // namespace

extern "C" {

int ql_abi_version(void) { return 113; }

const char *ql_strerror(int status) {
  switch (status) {
    case QL_OK: return "ok";
    case QL_EINVAL: return "invalid argument (null pointer, bad enum or non-positive size)";
    case QL_ESHAPE: return "unsupported or inconsistent shape";
    case QL_EALIGN: return "pointer not 16-byte aligned";
    case QL_EUNSUPPORTED: return "unsupported configuration";
    case QL_EWORKSPACE:
      return "workspace too small (qlora_linear_fwd_noalloc: the call needs more than its fixed "
             "workspace of QL_NOALLOC_WORKSPACE_BYTES)";
    case QL_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int ql_nf4_sizes(int64_t rows, int64_t cols, int32_t double_quant, size_t bytes_out[5]) {
  return ql_nf4_sizes_block(rows, cols, QL_NF4_BLOCK, double_quant, bytes_out);
}

int ql_nf4_sizes_block(int64_t rows, int64_t cols, int32_t block, int32_t double_quant,
                       size_t bytes_out[5]) {
  if (!bytes_out || rows <= 0 || cols <= 0 || (double_quant != 0 && double_quant != 1) ||
      (block != QL_NF4_BLOCK && block != QL_NF4_BLOCK_LARGE))
    return QL_EINVAL;
  const int64_t n = rows * cols;
  const int64_t nb = ceil_div(n, block);
  const int64_t nb2 = ceil_div(nb, QL_DQ_BLOCK);
  bytes_out[0] = (size_t)((n + 1) / 2);
  bytes_out[1] = double_quant ? 0 : (size_t)nb * 4;
  bytes_out[2] = double_quant ? (size_t)nb : 0;
  bytes_out[3] = double_quant ? (size_t)nb2 * 4 : 0;
  bytes_out[4] = double_quant ? 4 : 0;
  return QL_OK;
}

size_t ql_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r) {
  switch (op) {
    case QL_OP_QUANTIZE:
      if (N <= 0 || K <= 0) return 0;
      return quant_ws(N * K).total;
    case QL_OP_FWD:
      if (M <= 0 || N <= 0 || K <= 0 || r <= 0 || r > 128) return 0;
      return fwd_ws(M, N, K, r).total;
    case QL_OP_BWD:
      if (M <= 0 || N <= 0 || K <= 0 || r <= 0 || r > 128) return 0;
      return bwd_ws(M, N, K, r).total;
    default:
      return 0;
  }
}

int nf4_quantize(const void *w, int32_t w_dtype, const ql_nf4 *q, void *ws, size_t ws_bytes,
                 void *stream) {
  int st = check_nf4(q);
  if (st) return st;
  if (!w || check_dtype(w_dtype)) return QL_EINVAL;
  if (!aligned16(w)) return QL_EALIGN;
  const int64_t n = q->rows * q->cols;
  hipStream_t s = (hipStream_t)stream;
  if (!q->double_quant)
    return launch_nf4_quantize(w, w_dtype, n, q->block, q->packed, q->absmax, s);
  const QuantWs L = quant_ws(n);  // sized for blocks of 64, an upper bound for 128
  if (!ws || ws_bytes < L.total) return QL_EWORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return QL_EALIGN;
  uint8_t *base = (uint8_t *)ws;
  float *absmax = (float *)(base + L.absmax);
  unsigned long long *partial = (unsigned long long *)(base + L.partial);
  return launch_nf4_quantize_dq(w, w_dtype, n, q->block, q->packed, absmax, partial, q->absmax_q,
                                q->absmax_scale, q->absmax_mean, s);
}

int nf4_quantize_many(int32_t count, const void *const *w, int32_t w_dtype, const ql_nf4 *q,
                      void *ws, size_t ws_bytes, void *stream) {
  if (count < 0) return QL_EINVAL;
  if (count == 0) return QL_OK;
  if (!w || !q || check_dtype(w_dtype)) return QL_EINVAL;
  // every check before the first launch: an error enqueues nothing
  size_t need = 0;
  for (int i = 0; i < count; ++i) {
    const int st = check_nf4(&q[i]);
    if (st) return st;
    if (q[i].block != q[0].block || q[i].double_quant != q[0].double_quant) return QL_EINVAL;
    if (!w[i]) return QL_EINVAL;
    if (!aligned16(w[i])) return QL_EALIGN;
    if (q[i].double_quant) {
      const int64_t n = q[i].rows * q[i].cols;
      if ((n + q[i].block - 1) / q[i].block >= (int64_t(1) << 31)) return QL_EUNSUPPORTED;
      need += quant_ws(n).total;
    }
  }
  const bool dq = q[0].double_quant != 0;
  if (dq) {
    if (!ws || ws_bytes < need) return QL_EWORKSPACE;
    if (((uintptr_t)ws & (kAlign - 1)) != 0) return QL_EALIGN;
  }
  hipStream_t s = (hipStream_t)stream;
  uint8_t *base = (uint8_t *)ws;
  for (int i0 = 0; i0 < count; i0 += kQmMax) {
    const int c = std::min(kQmMax, count - i0);
    const void *wv[kQmMax];
    int64_t nv[kQmMax];
    uint8_t *pk[kQmMax];
    float *am[kQmMax], *sg[kQmMax], *mu[kQmMax];
    unsigned long long *pt[kQmMax];
    int8_t *qc[kQmMax];
    for (int j = 0; j < c; ++j) {
      const ql_nf4 &Q = q[i0 + j];
      wv[j] = w[i0 + j];
      nv[j] = Q.rows * Q.cols;
      pk[j] = Q.packed;
      if (dq) {  // this weight's part of the workspace: constants, then partial sums
        const QuantWs L = quant_ws(nv[j]);
        am[j] = (float *)(base + L.absmax);
        pt[j] = (unsigned long long *)(base + L.partial);
        base += L.total;
        qc[j] = Q.absmax_q;
        sg[j] = Q.absmax_scale;
        mu[j] = Q.absmax_mean;
      } else {
        am[j] = Q.absmax;
        pt[j] = nullptr;
        qc[j] = nullptr;
        sg[j] = mu[j] = nullptr;
      }
    }
    const int st = launch_nf4_quantize_many(c, wv, w_dtype, nv, q[0].block, dq, pk, am, pt, qc, sg,
                                            mu, s);
    if (st) return st;
  }
  return QL_OK;
}

int nf4_dequantize(const ql_nf4 *q, void *out, int32_t out_dtype, void *stream) {
  int st = check_nf4(q);
  if (st) return st;
  if (!out || check_dtype(out_dtype)) return QL_EINVAL;
  if (!aligned16(out)) return QL_EALIGN;
  return launch_nf4_dequantize(q->packed, q->rows * q->cols, scales_of(q), out, out_dtype,
                               (hipStream_t)stream);
}

// drop: LoRA dropout of the bypass input, with dscale = 1 / (1 - p); NULL
// for none.
static int linear_fwd(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                      const void *A, const void *B, int32_t lora_dtype, int32_t r, float alpha,
                      const Dropout *drop, float dscale, void *y, float *u_save, void *ws,
                      size_t ws_bytes, void *stream) {
  int st = check_linear_common(act_dtype, M, W, A, B, lora_dtype, r, alpha);
  if (st) return st;
  if (!x || !y) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(y) || (u_save && !aligned16(u_save))) return QL_EALIGN;
  const int64_t N = W->rows, K = W->cols;
  const FwdWs L = fwd_ws(M, N, K, r);
  if (!ws || ws_bytes < L.total) return QL_EWORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return QL_EALIGN;
  uint8_t *base = (uint8_t *)ws;
  float *u = u_save ? u_save : (float *)(base + L.u);
  float *rows_partial = (float *)(base + L.rows);
  hipStream_t s = (hipStream_t)stream;
  const float sc_lora = alpha / (float)r;
  const BlockScales sc = scales_of(W);
  if (act_dtype != QL_F32 && gemv_fwd_preferred(M, N, K))
    return launch_gemv_fwd(x, act_dtype, M, W->packed, sc, N, K, A, B, lora_dtype, r, sc_lora, y,
                           u_save, s, rows_partial, drop, dscale);
  if (act_dtype != QL_F32 && gemm_fwd_fused_preferred(M))
    return launch_gemm_fwd_fused(x, act_dtype, M, W->packed, sc, N, K, A, B, lora_dtype, r,
                                 sc_lora, y, u_save, s, rows_partial, drop, dscale);
  if (!drop && tiny_preferred(act_dtype, M, N, K, r))
    return launch_tiny_fwd(x, M, W->packed, sc, N, K, A, B, lora_dtype, r, sc_lora, y, u_save, s);
  st = launch_lora_rows_ws(x, act_dtype, M, K, A, lora_dtype, K, 1, r, drop ? dscale : 1.0f, u,
                           rows_partial, s, nullptr, drop);
  if (st) return st;
  if (act_dtype != QL_F32)
    return launch_gemm_fwd(x, act_dtype, M, W->packed, sc, N, K, u, B, lora_dtype, r, sc_lora, y,
                           s, rows_partial);
  return launch_simple_fwd(x, act_dtype, M, W->packed, sc, N, K, u, B, lora_dtype, r, sc_lora, y,
                           s);
}

int qlora_linear_fwd(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                     const void *A, const void *B, int32_t lora_dtype, int32_t r, float alpha,
                     void *y, float *u_save, void *ws, size_t ws_bytes, void *stream) {
  return linear_fwd(x, act_dtype, M, W, A, B, lora_dtype, r, alpha, nullptr, 1.0f, y, u_save, ws,
                    ws_bytes, stream);
}

// The device address of `scratch` on the current device, looked up on the
// first call per device (kMaxDevices at most).
static constexpr int kMaxDevices = 64;
static void *g_scratch[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];

static int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QL_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return QL_EUNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void *ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev]) return QL_EHIP;
  *out = g_scratch[dev];
  return QL_OK;
}

int qlora_linear_fwd_noalloc(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                             const void *A, const void *B, int32_t lora_dtype, int32_t r,
                             float alpha, void *y, float *u_save, void *stream) {
  int st = check_nf4(W);
  if (st) return st;
  if (M <= 0 || r <= 0 || r > 128) return QL_EINVAL;
  const size_t need = fwd_ws(M, W->rows, W->cols, r).total;
  if (need > (size_t)QL_NOALLOC_WORKSPACE_BYTES) return QL_EWORKSPACE;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  return linear_fwd(x, act_dtype, M, W, A, B, lora_dtype, r, alpha, nullptr, 1.0f, y, u_save, ws,
                    (size_t)QL_NOALLOC_WORKSPACE_BYTES, stream);
}

int qlora_linear_fwd_dropout(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                             const void *A, const void *B, int32_t lora_dtype, int32_t r,
                             float alpha, double dropout_p, uint64_t seed, void *y,
                             float *u_save, void *ws, size_t ws_bytes, void *stream) {
  Dropout d;
  float dscale;
  const int st = dropout_of(dropout_p, seed, d, dscale);
  if (st) return st;
  return linear_fwd(x, act_dtype, M, W, A, B, lora_dtype, r, alpha, dropout_p > 0.0 ? &d : nullptr,
                    dscale, y, u_save, ws, ws_bytes, stream);
}

int qlora_linear_fwd_u(const void *x, int32_t act_dtype, int64_t M, const ql_nf4 *W,
                       const float *u, const void *B, int32_t lora_dtype, int32_t r,
                       float alpha, void *y, void *stream) {
  // A is not read; B stands in for it in the shared argument check
  int st = check_linear_common(act_dtype, M, W, B, B, lora_dtype, r, alpha);
  if (st) return st;
  if (!x || !y || !u) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(u)) return QL_EALIGN;
  const int64_t N = W->rows, K = W->cols;
  hipStream_t s = (hipStream_t)stream;
  const float sc_lora = alpha / (float)r;
  const BlockScales sc = scales_of(W);
  if (act_dtype != QL_F32)
    return launch_gemm_fwd(x, act_dtype, M, W->packed, sc, N, K, u, B, lora_dtype, r, sc_lora, y,
                           s, nullptr);
  return launch_simple_fwd(x, act_dtype, M, W->packed, sc, N, K, u, B, lora_dtype, r, sc_lora, y,
                           s);
}

static int linear_bwd(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                      const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                      int32_t r, float alpha, const float *u_saved, void *dx, float *dA,
                      float *dB, void *ws, size_t ws_bytes, void *stream, bool accumulate,
                      const Dropout *drop = nullptr, float dscale = 1.0f) {
  int st = check_linear_common(act_dtype, M, W, A, B, lora_dtype, r, alpha);
  if (st) return st;
  if (!dy || !x || !dA || !dB) return QL_EINVAL;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(dA) || !aligned16(dB) ||
      (dx && !aligned16(dx)) || (u_saved && !aligned16(u_saved)))
    return QL_EALIGN;
  const int64_t N = W->rows, K = W->cols;
  const BwdWs L = bwd_ws(M, N, K, r);
  if (!ws || ws_bytes < L.total) return QL_EWORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return QL_EALIGN;
  uint8_t *base = (uint8_t *)ws;
  float *u = (float *)(base + L.u);
  float *g = (float *)(base + L.g);
  float *rows_partial = (float *)(base + L.rows);
  float *cols_partial = (float *)(base + L.cols);
  float *cols_partial2 = (float *)(base + L.cols2);
  hipStream_t s = (hipStream_t)stream;
  const float sc_lora = alpha / (float)r;
  const BlockScales sc = scales_of(W);
  if (!drop && tiny_preferred(act_dtype, M, N, K, r))
    return launch_tiny_bwd(dy, x, M, W->packed, sc, N, K, A, B, lora_dtype, r, sc_lora, u_saved,
                           dx, dA, dB, accumulate, s);
  if (u_saved) {
    u = const_cast<float *>(u_saved);
  } else {
    st = launch_lora_rows_ws(x, act_dtype, M, K, A, lora_dtype, K, 1, r, drop ? dscale : 1.0f, u,
                             rows_partial, s, nullptr, drop);
    if (st) return st;
  }
  // g = s dy B: Q(j, c) = B[c][j]
  st = launch_lora_rows_ws(dy, act_dtype, M, N, B, lora_dtype, 1, r, r, sc_lora, g, rows_partial, s);
  if (st) return st;
  // dB[n][j] = s sum_m dy[m][n] u[m][j] and dA[j][k] = sum_m g[m][j] x[m][k]
  // (x after dropout: keep / (1 - p) times x); without dropout both in one
  // launch
  ColsReduce red_dB, red_dA;
  if (!drop) {
    st = launch_lora_cols2(u, dy, N, sc_lora, true, dB, cols_partial, g, x, K, 1.0f, false, dA,
                           cols_partial2, M, r, act_dtype, s, accumulate, &red_dB, &red_dA);
    if (st) return st;
  } else {
    st = launch_lora_cols(u, M, r, dy, act_dtype, N, sc_lora, true, dB, cols_partial, s,
                          accumulate, nullptr, &red_dB);
    if (st) return st;
    st = launch_lora_cols(g, M, r, x, act_dtype, K, dscale, false, dA, cols_partial2, s,
                          accumulate, drop, &red_dA);
    if (st) return st;
  }
  st = launch_reduce_cols(red_dB, red_dA, s);
  if (st) return st;
  if (!dx) return QL_OK;
  if (act_dtype != QL_F32 && gemm_dx_supported(N, K))
    return launch_gemm_dx(dy, act_dtype, M, W->packed, sc, N, K, g, A, lora_dtype, r, dx, s,
                          rows_partial, drop, dscale);
  return launch_simple_dx(dy, act_dtype, M, W->packed, sc, N, K, g, A, lora_dtype, r, dx, s, drop,
                          dscale);
}

int qlora_linear_bwd(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                     const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                     int32_t r, float alpha, const float *u_saved, void *dx, float *dA,
                     float *dB, void *ws, size_t ws_bytes, void *stream) {
  return linear_bwd(dy, x, act_dtype, M, W, A, B, lora_dtype, r, alpha, u_saved, dx, dA, dB, ws,
                    ws_bytes, stream, false);
}

int qlora_linear_bwd_acc(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                         const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                         int32_t r, float alpha, const float *u_saved, void *dx, float *dA,
                         float *dB, void *ws, size_t ws_bytes, void *stream) {
  return linear_bwd(dy, x, act_dtype, M, W, A, B, lora_dtype, r, alpha, u_saved, dx, dA, dB, ws,
                    ws_bytes, stream, true);
}

int qlora_linear_bwd_dropout(const void *dy, const void *x, int32_t act_dtype, int64_t M,
                             const ql_nf4 *W, const void *A, const void *B, int32_t lora_dtype,
                             int32_t r, float alpha, double dropout_p, uint64_t seed,
                             const float *u_saved, void *dx, float *dA, float *dB,
                             int32_t accumulate, void *ws, size_t ws_bytes, void *stream) {
  Dropout d;
  float dscale;
  const int st = dropout_of(dropout_p, seed, d, dscale);
  if (st) return st;
  if (accumulate != 0 && accumulate != 1) return QL_EINVAL;
  return linear_bwd(dy, x, act_dtype, M, W, A, B, lora_dtype, r, alpha, u_saved, dx, dA, dB, ws,
                    ws_bytes, stream, accumulate == 1, dropout_p > 0.0 ? &d : nullptr, dscale);
}

int ql_dropout_mask(int64_t M, int64_t K, double dropout_p, uint64_t seed, uint8_t *keep,
                    void *stream) {
  Dropout d;
  float dscale;
  const int st = dropout_of(dropout_p, seed, d, dscale);
  if (st) return st;
  if (M <= 0 || K <= 0 || !keep) return QL_EINVAL;
  if (!aligned16(keep)) return QL_EALIGN;
  return launch_dropout_mask(M, K, d, keep, (hipStream_t)stream);
}

int ql_adamw_step(float *param, const float *grad, float *exp_avg, float *exp_avg_sq,
                  uint16_t *param_bf16, int64_t n, double lr, double beta1, double beta2,
                  double eps, double weight_decay, int64_t step, void *stream) {
  if (n < 0 || step < 1) return QL_EINVAL;
  if (n == 0) return QL_OK;
  if (!param || !grad || !exp_avg || !exp_avg_sq) return QL_EINVAL;
  if (!aligned16(param) || !aligned16(grad) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      (param_bf16 && ((uintptr_t)param_bf16 & 7) != 0))
    return QL_EALIGN;
  if (!(lr == lr) || !(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) ||
      !(eps > 0.0) || !(weight_decay == weight_decay))
    return QL_EINVAL;
  return launch_adamw(param, grad, exp_avg, exp_avg_sq, param_bf16, n, lr, beta1, beta2, eps,
                      weight_decay, step, (hipStream_t)stream);
}

}  // extern "C"
