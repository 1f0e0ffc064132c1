/*
 * nf4_oracle.c -- plain, slow, obviously-correct CPU reference for the QLoRA
 * quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the GPU
 * library; the codebook below is typed in from the pages on its own.
 *
 * Sources (the five pages on QLoRA; cited by page title and section):
 *   [ch26] "26. QLoRA and 4bit Quantization" (datawhalechina llm-algo-leetcode),
 *          Step 2 (NF4 codepoints, worked example 0.20 -> 0.161),
 *          Step 3 (forward y = x W^T + (x A^T) B^T * alpha/r),
 *          Step 4 (lookup table, dequantisation table[idx]*scale, tests).
 *   [ch22] "22. QLoRA and 4bit Quantization" (same site), Step 1 (gradient
 *          flows to x and LoRA only), Step 4 (uint8 holds two 4-bit values),
 *          engineering notes (blocks of 64 share one scale; double quant).
 *   [L9]   "QLoRA 4-bit quantised fine-tuning" (agentupdate.ai Gemma lesson 9),
 *          sec. 9.2.1 (block-wise: normalise each block to [-1,1], map to the
 *          nearest level, store 4-bit integers), sec. 9.2.2 (quantise the
 *          quantisation constants again to 8-bit integers).
 *   [gc4]  "QLoRA's three core techniques" (gufacode finetune chapter 4):
 *          double quantisation takes ~4.5 to ~4.127 bits per parameter.
 *
 * Precision: index and code decisions are taken in IEEE fp32 (the storage
 * precision of the constants); every matrix product accumulates in fp64.
 * Build with -ffp-contract=off so that no multiply-add is fused unless this
 * file says fmaf explicitly.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* [ch26] Step 4 / [ch22] Step 4: the 16-entry NF4 lookup table as printed
 * (index 7 is exactly zero, the ends are -1 and +1).  Stored as the fp32
 * values nearest to the printed decimals. */
static const float ORC_CB[16] = {
    -1.0f,  -0.696f, -0.525f, -0.395f, -0.284f, -0.185f, -0.091f, 0.0f,
    0.080f, 0.161f,  0.246f,  0.338f,  0.441f,  0.563f,  0.723f,  1.0f};

void orc_codebook(float *out16) { memcpy(out16, ORC_CB, sizeof(ORC_CB)); }

/* [ch26] Step 2, [L9] 9.2.1: map a normalised value to the nearest codepoint.
 * Distances are taken in fp64, where v - cb[i] is exact for every v close
 * enough to a midpoint to matter; equal distances resolve to the lower index
 * (strict '<' keeps the first minimum). */
int orc_nearest_index(float v) {
  int best = 0;
  double bd = fabs((double)v - (double)ORC_CB[0]);
  for (int i = 1; i < 16; ++i) {
    double d = fabs((double)v - (double)ORC_CB[i]);
    if (d < bd) {
      bd = d;
      best = i;
    }
  }
  return best;
}

/* Block-wise NF4 quantisation of a flattened tensor of n fp32 values
 * ([L9] 9.2.1; [ch22] notes: a block of 64 shares one scale).
 * Block b covers elements [b*block, min(n, (b+1)*block)).
 *   absmax[b] = max |w| over the block (the scale that makes [-1,1] exact)
 *   v = w / absmax[b]   (fp32, correctly rounded division)
 *   idx = nearest codepoint of v; an all-zero block codes every element as 7.
 * Packing ([ch22] Step 4: two 4-bit values per uint8): element 2j goes to the
 * high nibble of byte j, element 2j+1 to the low nibble; with odd n the last
 * low nibble is 0.  block must be even so blocks never share a byte. */
void orc_nf4_quantize(const float *w, int64_t n, int32_t block,
                      uint8_t *packed, float *absmax) {
  int64_t nb = (n + block - 1) / block;
  memset(packed, 0, (size_t)((n + 1) / 2));
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * block, hi = lo + block < n ? lo + block : n;
    float a = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float m = fabsf(w[i]);
      if (m > a) a = m;
    }
    absmax[b] = a;
    for (int64_t i = lo; i < hi; ++i) {
      int idx = 7;
      if (a != 0.0f) {
        float v = w[i] / a;
        idx = orc_nearest_index(v);
      }
      if ((i & 1) == 0)
        packed[i >> 1] = (uint8_t)(packed[i >> 1] | (idx << 4));
      else
        packed[i >> 1] = (uint8_t)(packed[i >> 1] | idx);
    }
  }
}

/* Unpack the 4-bit index of element i (inverse of the packing above). */
int orc_unpack_index(const uint8_t *packed, int64_t i) {
  uint8_t byte = packed[i >> 1];
  return (i & 1) == 0 ? (byte >> 4) : (byte & 15);
}

/* Double quantisation of the block constants ([L9] 9.2.2: the constants are
 * quantised again to 8-bit integers; [gc4]: 4.5 -> ~4.127 bits/param, which
 * is 8-bit codes plus one fp32 scale per 256 constants plus one fp32 mean).
 * mu is the per-tensor mean of the constants (computed by the caller from the
 * exact sum).  For constant block c = [c*block2, ...):
 *   d_j = absmax_j - mu                       (fp32)
 *   sigma_c = max_j |d_j| / 127               (fp32)
 *   q_j = clamp(round_half_even(d_j / sigma_c), -127, 127), 0 when sigma_c == 0
 */
void orc_dq_codes(const float *absmax, int64_t nb, float mu, int32_t block2,
                  int8_t *q, float *sigma) {
  int64_t nb2 = (nb + block2 - 1) / block2;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nb2; ++c) {
    int64_t lo = c * block2, hi = lo + block2 < nb ? lo + block2 : nb;
    float amax = 0.0f;
    for (int64_t j = lo; j < hi; ++j) {
      float d = absmax[j] - mu;
      if (fabsf(d) > amax) amax = fabsf(d);
    }
    float s = amax / 127.0f;
    sigma[c] = s;
    for (int64_t j = lo; j < hi; ++j) {
      float d = absmax[j] - mu;
      int code = 0;
      if (s != 0.0f) {
        float t = nearbyintf(d / s); /* default mode: ties to even */
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        code = (int)t;
      }
      q[j] = (int8_t)code;
    }
  }
}

/* Reconstruct one block constant: a' = code * sigma + mu with one rounding
 * (fmaf), or the stored fp32 absmax when there is no double quantisation. */
static float orc_block_scale(int64_t b, const float *absmax, const int8_t *q,
                             const float *sigma, float mu, int32_t block2) {
  if (absmax) return absmax[b];
  return fmaf((float)q[b], sigma[b / block2], mu);
}

/* Dequantisation ([ch26] Step 4: table[idx] * scale; [ch22] Step 3: restored
 * to a 16-bit float at the moment of the forward).  out[i] = fp32 product
 * cb[idx_i] * a'_{block(i)}.  Pass absmax for the single-level form, or
 * absmax == NULL with (q, sigma, mu, block2) for the double-quantised form. */
void orc_nf4_dequantize(const uint8_t *packed, int64_t n, int32_t block,
                        const float *absmax, const int8_t *q,
                        const float *sigma, float mu, int32_t block2,
                        float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t b = i / block;
    float a = orc_block_scale(b, absmax, q, sigma, mu, block2);
    out[i] = ORC_CB[orc_unpack_index(packed, i)] * a;
  }
}

/* fp32 -> bfloat16 with round-to-nearest-even on the bit pattern (finite
 * inputs; NaN is out of scope). */
void orc_round_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    out[i] = (uint16_t)(u >> 16);
  }
}

/* fp32 -> IEEE 754 binary16 bit pattern, round to nearest, ties to even,
 * from the format's definition: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits.  A finite x with |x| in [2^e, 2^(e+1)), e >= -14, is
 * m 2^(e-10) with m = rint(|x| 2^(10-e)) in [1024, 2048] (m = 2048 carries
 * into the next binade); |x| < 2^-14 is the subnormal m 2^-24 with
 * m = rint(|x| 2^24) (m = 1024 is the smallest normal, whose bit pattern is
 * the same integer).  Exponents past 15 are infinity (|x| >= 65520).  Every
 * scaling is by a power of two, exact in double; rint rounds half to even
 * in the default rounding mode.  (finite inputs; NaN is out of scope) */
static uint16_t orc_f16_bits(float x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  const double a = fabs((double)x);
  if (a < ldexp(1.0, -14)) return sign | (uint16_t)rint(ldexp(a, 24));
  int e;
  frexp(a, &e);  /* a = f 2^e, f in [0.5, 1): the binade exponent is e - 1 */
  e -= 1;
  double m = rint(ldexp(a, 10 - e));
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e > 15) return sign | 0x7C00u;
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024);
}

void orc_round_f16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_bits(in[i]);
}

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), written from
 * its definition there: a 4-word counter and a 2-word key; one round maps
 * (c0, c1, c2, c3) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
 * lo(M0 c0)) with the multipliers M0 = 0xD2511F53, M1 = 0xCD9E8D57; between
 * rounds the key is bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85);
 * 10 rounds.  The pages name LoRA dropout without saying how its mask is
 * drawn; this generator is the reading taken (see the dropout mask below). */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* LoRA dropout mask over the activations x [M, K] (the pages' LoraConfig
 * lora_dropout: dropout on the bypass input, inverted scaling 1/(1-p)).
 * Element e = m K + k takes word e % 4 of Philox4x32-10 at counter
 * (e / 4 low, e / 4 high, 0, 0) with key (seed low, seed high), and is kept
 * when that word >= threshold (threshold = floor(p 2^32)). */
void orc_dropout_keep(int64_t M, int64_t K, uint32_t threshold, uint64_t seed, uint8_t *keep) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  const int64_t n = M * K;
#pragma omp parallel for schedule(static)
  for (int64_t grp = 0; grp < (n + 3) / 4; ++grp) {
    const uint32_t ctr[4] = {(uint32_t)grp, (uint32_t)((uint64_t)grp >> 32), 0u, 0u};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i < n) keep[4 * grp + i] = w[i] >= threshold ? 1 : 0;
  }
}

/* Forward of the layer ([ch26] Step 3 / Step 4 answer):
 *   u = (d .* x) A^T          [M, r]
 *   y = x W^T + s * u B^T     [M, N],  s = alpha / r
 * x [M,K], w [N,K] (the dequantised weight), A [r,K], B [N,r]; d [M,K] the
 * dropout multipliers of the bypass input (0 or 1/(1-p)), or NULL for none.
 * All products accumulate in fp64 in index order.  u may be NULL. */
void orc_linear_fwd(int64_t M, int64_t N, int64_t K, int32_t r, double s,
                    const double *x, const float *w, const double *A,
                    const double *B, const double *d, double *y, double *u_out) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const double *xm = x + m * K;
    const double *dm = d ? d + m * K : NULL;
    double u[512];
    for (int32_t j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += (dm ? dm[k] * xm[k] : xm[k]) * A[j * K + k];
      u[j] = acc;
      if (u_out) u_out[m * r + j] = acc;
    }
    for (int64_t nn = 0; nn < N; ++nn) {
      const float *wn = w + nn * K;
      double base = 0.0;
      for (int64_t k = 0; k < K; ++k) base += xm[k] * (double)wn[k];
      double lora = 0.0;
      for (int32_t j = 0; j < r; ++j) lora += u[j] * B[nn * r + j];
      y[m * N + nn] = base + s * lora;
    }
  }
}

/* Backward of the layer ([ch22] Step 1 item 4 and [ch26] Step 4 tests: the
 * gradient reaches x, A and B; the frozen base gets none).  With the
 * dropped input xd = d .* x (xd = x when d is NULL), u = xd A^T and
 * g = s * dy B:
 *   dB = s * dy^T u          [N, r]
 *   dA = g^T xd              [r, K]
 *   dx = dy W + d .* (g A)   [M, K]
 * dx is produced only for the rows listed in rows[0..n_rows) (all rows when
 * rows == NULL), into dx[i*K ...] for the i-th listed row; dx may be NULL.
 * Work buffers u_buf and g_buf hold M*r doubles each.  Every sum runs over
 * its contraction index in increasing order; the loops are only nested so
 * that the inner loop walks memory contiguously. */
#define ORC_CHUNK 64
void orc_linear_bwd(int64_t M, int64_t N, int64_t K, int32_t r, double s,
                    const double *x, const float *w, const double *A,
                    const double *B, const double *d, const double *dy, const int64_t *rows,
                    int64_t n_rows, double *dx, double *dA, double *dB,
                    double *u_buf, double *g_buf) {
#define ORC_XD(m, k) (d ? d[(m) * K + (k)] * x[(m) * K + (k)] : x[(m) * K + (k)])
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int32_t j = 0; j < r; ++j) {
      double au = 0.0;
      for (int64_t k = 0; k < K; ++k) au += ORC_XD(m, k) * A[j * K + k];
      u_buf[m * r + j] = au;
      double ag = 0.0;
      for (int64_t nn = 0; nn < N; ++nn) ag += dy[m * N + nn] * B[nn * r + j];
      g_buf[m * r + j] = s * ag;
    }
  }
  /* dB[n][j] = s * sum_m dy[m][n] u[m][j] */
  int64_t ncn = (N + ORC_CHUNK - 1) / ORC_CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < ncn; ++c) {
    int64_t n0 = c * ORC_CHUNK, n1 = n0 + ORC_CHUNK < N ? n0 + ORC_CHUNK : N;
    for (int64_t nn = n0; nn < n1; ++nn)
      for (int32_t j = 0; j < r; ++j) dB[nn * r + j] = 0.0;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t nn = n0; nn < n1; ++nn) {
        double d = dy[m * N + nn];
        for (int32_t j = 0; j < r; ++j) dB[nn * r + j] += d * u_buf[m * r + j];
      }
    for (int64_t nn = n0; nn < n1; ++nn)
      for (int32_t j = 0; j < r; ++j) dB[nn * r + j] = s * dB[nn * r + j];
  }
  /* dA[j][k] = sum_m g[m][j] x[m][k] */
  int64_t nck = (K + ORC_CHUNK - 1) / ORC_CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nck; ++c) {
    int64_t k0 = c * ORC_CHUNK, k1 = k0 + ORC_CHUNK < K ? k0 + ORC_CHUNK : K;
    for (int32_t j = 0; j < r; ++j)
      for (int64_t k = k0; k < k1; ++k) dA[j * K + k] = 0.0;
    for (int64_t m = 0; m < M; ++m)
      for (int32_t j = 0; j < r; ++j) {
        double gv = g_buf[m * r + j];
        for (int64_t k = k0; k < k1; ++k) dA[j * K + k] += gv * ORC_XD(m, k);
      }
  }
  if (!dx) return;
  /* dx[m][k] = sum_n dy[m][n] w[n][k] + sum_j g[m][j] A[j][k] */
  int64_t nr = rows ? n_rows : M;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nr; ++i) {
    int64_t m = rows ? rows[i] : i;
    const double *dym = dy + m * N;
    double *dxi = dx + i * K;
    for (int64_t k = 0; k < K; ++k) dxi[k] = 0.0;
    for (int64_t nn = 0; nn < N; ++nn) {
      double d = dym[nn];
      const float *wn = w + nn * K;
      for (int64_t k = 0; k < K; ++k) dxi[k] += d * (double)wn[k];
    }
    for (int64_t k = 0; k < K; ++k) {
      double lora = 0.0;
      for (int32_t j = 0; j < r; ++j) lora += g_buf[m * r + j] * A[j * K + k];
      dxi[k] = dxi[k] + (d ? d[m * K + k] * lora : lora);
    }
  }
#undef ORC_XD
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of host threads the parallel loops above use (reported with the
 * CPU baseline timing). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of host threads of the parallel loops (timing only: no
 * result depends on it). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* One AdamW step over n fp32 parameters, in place.  [gc4] "显存计算实战" and
 * "分页优化器": the LoRA factors are trained with AdamW (torch.optim.AdamW,
 * lr 2e-4) holding fp32 moments, 8 bytes per trainable parameter; [L9] 9.4:
 * two states (momentum and variance) per parameter.  The pages do not write
 * the update out; it is the published AdamW definition (decoupled weight
 * decay, bias-corrected moments), every operation an fp32 rounding, none
 * fused, in this order:
 *   p  = p * decay                         decay = fp32(1 - lr * wd)
 *   m  = b1 * m + (1 - b1) * g
 *   v  = b2 * v + (1 - b2) * (g * g)
 *   p  = p - step_size * (m / (sqrt(v) / bc2_sqrt + eps))
 * with the scalars computed once in fp64 and rounded to fp32 by the caller:
 *   step_size = lr / (1 - b1^t),  bc2_sqrt = sqrt(1 - b2^t).
 * p_bf16 (optional) receives the round-to-nearest-even bf16 of the new p. */
void orc_adamw_step(float *p, const float *g, float *m, float *v, uint16_t *p_bf16, int64_t n,
                    float decay, float b1, float omb1, float b2, float omb2, float eps,
                    float step_size, float bc2_sqrt) {
  for (int64_t i = 0; i < n; ++i) {
    float pi = p[i] * decay;
    float mi = b1 * m[i] + omb1 * g[i];
    float gg = g[i] * g[i];
    float vi = b2 * v[i] + omb2 * gg;
    float denom = sqrtf(vi) / bc2_sqrt + eps;
    float upd = mi / denom;
    pi = pi - step_size * upd;
    p[i] = pi;
    m[i] = mi;
    v[i] = vi;
    if (p_bf16) { /* round to nearest even, as orc_round_bf16 */
      uint32_t u;
      memcpy(&u, &pi, 4);
      u += 0x7FFFu + ((u >> 16) & 1u);
      p_bf16[i] = (uint16_t)(u >> 16);
    }
  }
}
