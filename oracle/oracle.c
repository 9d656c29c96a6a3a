/*
 * CPU oracle for the per-denoising-step quantized GEMM stream.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The product
 * path (libdllm) never links, loads or calls it, and shares no code with it.
 *
 * What it computes (mojo-dllm Development plan, "Compute design"): each linear
 * layer multiplies L per-token Q8_K activation rows (int8 quants, one f32 scale
 * per 256 values, int sums per 16) by GGUF Q4_K / Q6_K weight rows; the LM head
 * runs only on the masked rows of the current block (same section, last
 * bullet; README "How it works", "Logits only where the sampler looks").
 *
 * The pages name the GGUF block types but never print their byte layouts.
 * The layouts used here are the public GGUF definitions, restated from the
 * format description (Q4_K: 144-byte super-block, Q6_K: 210 bytes, Q8_K: 292
 * bytes).  The method reaches exactly the plain result y = W_hat . X_hat^T of
 * the dequantized operands, so the oracle is that definition: every block is
 * decoded exactly into f64 and every dot product is summed in f64 in
 * ascending index order.  The Q8_K quantizer is an integer-producing decision
 * made in f32, so it is evaluated in f32 exactly as the format defines it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (no SIMD
 * intrinsics; threads only split output rows).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ---- IEEE binary16 -> f64, by its bits (exact) ------------------------- */
double oracle_f16_to_f64(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 31;
  const int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY; /* never produced by the generator */
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static float rdf32(const uint8_t *p) {
  float f;
  memcpy(&f, p, 4);
  return f;
}

/* ---- Q4_K super-block fields ------------------------------------------- */
/* Bytes: [0,2) f16 d, [2,4) f16 dmin, [4,16) twelve bytes holding eight 6-bit
 * scales and eight 6-bit mins, [16,144) 128 bytes of 4-bit quants.
 * Scales/mins: sub-blocks 0..3 keep theirs in the low 6 bits of bytes 0..3
 * (scale) and 4..7 (min); sub-blocks 4..7 keep the low 4 bits in the two
 * nibbles of bytes 8..11 and the top 2 bits in the spare top bits of bytes
 * 0..3 (scale) and 4..7 (min).
 * Quants: sub-block j (32 weights) lives in the 32-byte run 32*(j/2), low
 * nibbles for even j, high nibbles for odd j. */
void oracle_q4k_fields(const uint8_t *b, double *d, double *dmin, int sc[8],
                       int mn[8], int u[256]) {
  const uint8_t *S = b + 4;
  const uint8_t *qs = b + 16;
  *d = oracle_f16_to_f64(rd16(b));
  *dmin = oracle_f16_to_f64(rd16(b + 2));
  for (int j = 0; j < 8; ++j) {
    if (j < 4) {
      sc[j] = S[j] & 63;
      mn[j] = S[j + 4] & 63;
    } else {
      sc[j] = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
      mn[j] = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
  }
  for (int i = 0; i < 256; ++i) {
    const int j = i / 32, l = i % 32;
    const uint8_t byte = qs[32 * (j / 2) + l];
    u[i] = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
  }
}

/* ---- Q6_K super-block fields ------------------------------------------- */
/* Bytes: [0,128) low 4 bits of the quants, [128,192) high 2 bits,
 * [192,208) sixteen int8 scales (one per 16 weights), [208,210) f16 d.
 * Weight i: half h = i/128, r = i%128, quarter k = r/32, l = r%32.  Low 4 bits
 * from byte 64h + 32(k&1) + l (low nibble for k<2, high nibble for k>=2); high
 * 2 bits are bits 2k..2k+1 of byte 128 + 32h + l.  The 6-bit quant q is in
 * [0,63] and the weight is d * scale[i/16] * (q - 32). */
void oracle_q6k_fields(const uint8_t *b, double *d, int sc[16], int q[256]) {
  const uint8_t *ql = b, *qh = b + 128;
  const int8_t *s = (const int8_t *)(b + 192);
  *d = oracle_f16_to_f64(rd16(b + 208));
  for (int g = 0; g < 16; ++g) sc[g] = s[g];
  for (int i = 0; i < 256; ++i) {
    const int h = i / 128, r = i % 128, k = r / 32, l = r % 32;
    const uint8_t lb = ql[64 * h + 32 * (k & 1) + l];
    const int low4 = (k < 2) ? (lb & 15) : (lb >> 4);
    const int high2 = (qh[32 * h + l] >> (2 * k)) & 3;
    q[i] = low4 | (high2 << 4);
  }
}

static int block_bytes(int qtype) {
  if (qtype == ORACLE_Q4_K) return 144;
  if (qtype == ORACLE_Q6_K) return 210;
  return 0;
}

/* Exact f64 values of one weight super-block. */
static int decode_block_f64(int qtype, const uint8_t *b, double *w) {
  if (qtype == ORACLE_Q4_K) {
    double d, dmin;
    int sc[8], mn[8], u[256];
    oracle_q4k_fields(b, &d, &dmin, sc, mn, u);
    for (int i = 0; i < 256; ++i) {
      const int j = i / 32;
      w[i] = d * sc[j] * u[i] - dmin * mn[j];
    }
    return 0;
  }
  if (qtype == ORACLE_Q6_K) {
    double d;
    int sc[16], q[256];
    oracle_q6k_fields(b, &d, sc, q);
    for (int i = 0; i < 256; ++i) w[i] = d * sc[i / 16] * (q[i] - 32);
    return 0;
  }
  return -1;
}

int oracle_decode_rows(int qtype, const uint8_t *w, int64_t N, int64_t K,
                       double *out) {
  const int bb = block_bytes(qtype);
  if (!bb || K % 256) return -1;
  const int64_t nsb = K / 256;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t s = 0; s < nsb; ++s)
      decode_block_f64(qtype, w + (n * nsb + s) * bb, out + n * K + s * 256);
  return 0;
}

/* ---- shared decoded form (Development plan, "Compute design", 2nd bullet):
 * unsigned bytes, an int16 scale per 16 and an f32 offset per 16, plus the
 * super-block f32 factor D so that w_i = D * sc16[i/16] * u_i + off[i/16].
 * Layout of one 356-byte record: f32 D | f32 off[16] | i16 sc16[16] | u8 u[256].
 *   Q4_K: u = 4-bit quant, sc16[g] = scale[g/2], off[g] = -(f32(dmin)*min[g/2]).
 *   Q6_K: u = 6-bit quant q, sc16[g] = scale[g], off[g] = -(32*f32(d)*scale[g]).
 * Every field is exact in its type. */
int oracle_decode_shared(int qtype, const uint8_t *w, int64_t nsb, uint8_t *out) {
  const int bb = block_bytes(qtype);
  if (!bb) return -1;
  for (int64_t s = 0; s < nsb; ++s) {
    const uint8_t *b = w + s * bb;
    uint8_t *o = out + s * 356;
    float D, off[16];
    int16_t sc16[16];
    uint8_t u8[256];
    if (qtype == ORACLE_Q4_K) {
      double d, dmin;
      int sc[8], mn[8], u[256];
      oracle_q4k_fields(b, &d, &dmin, sc, mn, u);
      D = (float)d;
      const float fdmin = (float)dmin;
      for (int g = 0; g < 16; ++g) {
        sc16[g] = (int16_t)sc[g / 2];
        off[g] = -(fdmin * (float)mn[g / 2]);
      }
      for (int i = 0; i < 256; ++i) u8[i] = (uint8_t)u[i];
    } else {
      double d;
      int sc[16], q[256];
      oracle_q6k_fields(b, &d, sc, q);
      D = (float)d;
      for (int g = 0; g < 16; ++g) {
        sc16[g] = (int16_t)sc[g];
        off[g] = -(32.0f * D * (float)sc[g]);
      }
      for (int i = 0; i < 256; ++i) u8[i] = (uint8_t)q[i];
    }
    memcpy(o, &D, 4);
    memcpy(o + 4, off, 64);
    memcpy(o + 68, sc16, 32);
    memcpy(o + 100, u8, 256);
  }
  return 0;
}

/* ---- Q8_K quantization, f32 as the format defines it ------------------- */
/* Per 256-value block: the pivot is the first value of largest magnitude;
 * iscale = -127/pivot (f32, correctly rounded); q_i = min(127, round-half-even
 * (iscale * x_i)) with the product rounded to f32 first; d = 1/iscale; the 16
 * bsums are the int sums of each run of 16 quants.  An all-zero block gives
 * d = 0 and all-zero quants and sums.  Record: f32 d | int8 q[256] |
 * int16 bsums[16]. */
static void quantize_block_q8k(const float *x, uint8_t *o) {
  float amax = 0.0f, pivot = 0.0f;
  for (int i = 0; i < 256; ++i) {
    const float a = fabsf(x[i]);
    if (a > amax) {
      amax = a;
      pivot = x[i];
    }
  }
  int8_t q[256];
  int16_t bs[16];
  float d;
  if (amax == 0.0f) {
    d = 0.0f;
    memset(q, 0, sizeof q);
    memset(bs, 0, sizeof bs);
  } else {
    const float iscale = -127.0f / pivot;
    for (int i = 0; i < 256; ++i) {
      const float p = iscale * x[i];
      int v = (int)rintf(p);
      if (v > 127) v = 127;
      q[i] = (int8_t)v;
    }
    for (int g = 0; g < 16; ++g) {
      int s = 0;
      for (int t = 0; t < 16; ++t) s += q[16 * g + t];
      bs[g] = (int16_t)s;
    }
    d = 1.0f / iscale;
  }
  memcpy(o, &d, 4);
  memcpy(o + 4, q, 256);
  memcpy(o + 260, bs, 32);
}

int oracle_quantize_q8k(const float *x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t *out) {
  if (K % 256 || ldx < K) return -1;
  const int64_t nsb = K / 256;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t s = 0; s < nsb; ++s)
      quantize_block_q8k(x + m * ldx + s * 256, out + (m * nsb + s) * 292);
  return 0;
}

/* x_hat = d * q, exact in f64. */
int oracle_dequant_q8k(const uint8_t *xq, int64_t M, int64_t K, double *out) {
  if (K % 256) return -1;
  const int64_t nsb = K / 256;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t s = 0; s < nsb; ++s) {
      const uint8_t *b = xq + (m * nsb + s) * 292;
      const double d = (double)rdf32(b);
      const int8_t *q = (const int8_t *)(b + 4);
      for (int i = 0; i < 256; ++i) out[m * K + s * 256 + i] = d * q[i];
    }
  return 0;
}

/* ---- GEMM: y[m][n] = sum_i w_hat[n][i] * x_hat[m][i], f64, ascending i ---- */
typedef struct {
  int qtype;
  const uint8_t *w;
  int64_t N, K, M;
  const double *xh; /* [M][K] dequantized activations */
  double *y;        /* [M][N] */
  int64_t n0, n1;
} gemm_job;

static void *gemm_worker(void *arg) {
  gemm_job *j = (gemm_job *)arg;
  const int bb = block_bytes(j->qtype);
  const int64_t nsb = j->K / 256;
  double *wrow = (double *)malloc(sizeof(double) * j->K);
  for (int64_t n = j->n0; n < j->n1; ++n) {
    for (int64_t s = 0; s < nsb; ++s)
      decode_block_f64(j->qtype, j->w + (n * nsb + s) * bb, wrow + s * 256);
    for (int64_t m = 0; m < j->M; ++m) {
      const double *xr = j->xh + m * j->K;
      double acc = 0.0;
      for (int64_t i = 0; i < j->K; ++i) acc += wrow[i] * xr[i];
      j->y[m * j->N + n] = acc;
    }
  }
  free(wrow);
  return NULL;
}

static int run_threads(gemm_job *base, int64_t N, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > N) nthreads = (int)(N > 0 ? N : 1);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  gemm_job *jobs = (gemm_job *)malloc(sizeof(gemm_job) * nthreads);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *base;
    jobs[t].n0 = N * t / nthreads;
    jobs[t].n1 = N * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
  return 0;
}

int oracle_gemm(int qtype, const uint8_t *w, int64_t N, int64_t K,
                const uint8_t *xq, int64_t M, double *y, int nthreads) {
  if (!block_bytes(qtype) || K % 256 || N < 0 || M < 0) return -1;
  double *xh = (double *)malloc(sizeof(double) * (M * K > 0 ? M * K : 1));
  oracle_dequant_q8k(xq, M, K, xh);
  gemm_job base = {qtype, w, N, K, M, xh, y, 0, 0};
  run_threads(&base, N, nthreads);
  free(xh);
  return 0;
}

/* Individual outputs y[mi[t]][ni[t]] for sampled checks at full size. */
int oracle_gemm_sample(int qtype, const uint8_t *w, int64_t N, int64_t K,
                       const uint8_t *xq, int64_t M, const int64_t *mi,
                       const int64_t *ni, int64_t count, double *out) {
  const int bb = block_bytes(qtype);
  if (!bb || K % 256) return -1;
  const int64_t nsb = K / 256;
  double *wrow = (double *)malloc(sizeof(double) * K);
  double *xrow = (double *)malloc(sizeof(double) * K);
  for (int64_t t = 0; t < count; ++t) {
    if (mi[t] < 0 || mi[t] >= M || ni[t] < 0 || ni[t] >= N) {
      free(wrow);
      free(xrow);
      return -2;
    }
    for (int64_t s = 0; s < nsb; ++s)
      decode_block_f64(qtype, w + (ni[t] * nsb + s) * bb, wrow + s * 256);
    oracle_dequant_q8k(xq + mi[t] * nsb * 292, 1, K, xrow);
    double acc = 0.0;
    for (int64_t i = 0; i < K; ++i) acc += wrow[i] * xrow[i];
    out[t] = acc;
  }
  free(wrow);
  free(xrow);
  return 0;
}

/* ---- per-16 integer partial dots of the shared form ------------------- */
/* P[m][n][sb][g] = sum_{t<16} u[n][256 sb + 16 g + t] * q[m][256 sb + 16 g + t],
 * with u the unsigned shared-form quant (Q4_K 4-bit, Q6_K 6-bit). */
int oracle_partials(int qtype, const uint8_t *w, int64_t N, int64_t K,
                    const uint8_t *xq, int64_t M, int32_t *P) {
  const int bb = block_bytes(qtype);
  if (!bb || K % 256) return -1;
  const int64_t nsb = K / 256;
  int u[256];
  for (int64_t n = 0; n < N; ++n)
    for (int64_t s = 0; s < nsb; ++s) {
      const uint8_t *b = w + (n * nsb + s) * bb;
      if (qtype == ORACLE_Q4_K) {
        double d, dmin;
        int sc[8], mn[8];
        oracle_q4k_fields(b, &d, &dmin, sc, mn, u);
      } else {
        double d;
        int sc[16];
        oracle_q6k_fields(b, &d, sc, u);
      }
      for (int64_t m = 0; m < M; ++m) {
        const int8_t *q = (const int8_t *)(xq + (m * nsb + s) * 292 + 4);
        for (int g = 0; g < 16; ++g) {
          int64_t acc = 0;
          for (int t = 0; t < 16; ++t) acc += (int64_t)u[16 * g + t] * q[16 * g + t];
          P[((m * N + n) * nsb + s) * 16 + g] = (int32_t)acc;
        }
      }
    }
  return 0;
}

/* ---- masked-row LM head ------------------------------------------------ */
/* Gather rows[r] of h (f32, leading dimension ldh), quantize each to Q8_K,
 * multiply by the output matrix (f64 logits), and take the per-row argmax,
 * lowest index on ties. */
int oracle_lmhead(int qtype, const uint8_t *w, int64_t N, int64_t K,
                  const float *h, int64_t M, int64_t ldh, const int32_t *rows,
                  int64_t n_rows, double *logits, int32_t *argmax, int nthreads) {
  if (!block_bytes(qtype) || K % 256 || ldh < K) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -2;
  const int64_t nsb = K / 256;
  uint8_t *xq = (uint8_t *)calloc((size_t)(n_rows * nsb * 292 + 1), 1);
  for (int64_t r = 0; r < n_rows; ++r)
    oracle_quantize_q8k(h + (int64_t)rows[r] * ldh, 1, K, K, xq + r * nsb * 292);
  oracle_gemm(qtype, w, N, K, xq, n_rows, logits, nthreads);
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t best = 0;
    for (int64_t n = 1; n < N; ++n)
      if (logits[r * N + n] > logits[r * N + best]) best = n;
    argmax[r] = (int32_t)best;
  }
  free(xq);
  return 0;
}

/* ---- confidence of the greedy pick ------------------------------------- */
/* Per logit row (the masked positions of a step): the log-sum-exp of the
 * row, lse = m + log(sum_n exp(l_n - m)) with m = max_n l_n, and the softmax
 * probability of the argmax token, exp(m - lse) = 1 / sum_n exp(l_n - m).
 * The pages list softmax, log-softmax and argmax among the sampling
 * primitives and give LLaDA low-confidence remasking, whose confidence of a
 * committed token is its softmax probability.  Sums in f64, ascending n. */
int oracle_softmax_stats(const double *logits, int64_t n_rows, int64_t N, double *lse, double *p_argmax) {
  if (N <= 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    const double *l = logits + r * N;
    double m = l[0];
    for (int64_t n = 1; n < N; ++n)
      if (l[n] > m) m = l[n];
    double s = 0.0;
    for (int64_t n = 0; n < N; ++n) s += exp(l[n] - m);
    lse[r] = m + log(s);
    p_argmax[r] = 1.0 / s;
  }
  return 0;
}

/* ---- fused producers of the quantized activations ---------------------- */
/* The pages' layer runs RMSNorm before the QKV and MLP projections (eps 1e-5
 * for LLaDA) and a SwiGLU MLP, and list fused normalization among the next
 * goals.  These are the two producers fused with the Q8_K quantizer.
 *
 * RMSNorm -> Q8_K, per row of x (K values) with norm weight g[K]:
 *   r = f32(1 / sqrt(sum_k x_k^2 / K + eps))   (squares exact in f64, the sum
 *                                              in f64 ascending, sqrt and
 *                                              division in f64, one rounding)
 *   z_k = f32(x_k * g_k)
 *   the Q8_K blocks of z (codes and bsums), with each block's d replaced by
 *   f32(r * d_z): the blocks of RMSNorm(x) = r * z with the common factor r
 *   moved into the block scale, so the codes do not depend on r.
 * dmax[m] (optional): the row's largest |d|. */
int oracle_rmsnorm_quantize_q8k(const float *x, int64_t M, int64_t K, int64_t ldx, const float *g, float eps,
                                uint8_t *out, float *dmax) {
  if (K % 256 || ldx < K) return -1;
  const int64_t nsb = K / 256;
  float *z = (float *)malloc(sizeof(float) * (size_t)K);
  for (int64_t m = 0; m < M; ++m) {
    const float *xr = x + m * ldx;
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) ss += (double)xr[k] * (double)xr[k];
    const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    for (int64_t k = 0; k < K; ++k) z[k] = xr[k] * g[k];
    float mx = 0.0f;
    for (int64_t s = 0; s < nsb; ++s) {
      uint8_t *b = out + (m * nsb + s) * 292;
      quantize_block_q8k(z + s * 256, b);
      const float d = r * rdf32(b);
      memcpy(b, &d, 4);
      if (fabsf(d) > mx) mx = fabsf(d);
    }
    if (dmax) dmax[m] = mx;
  }
  free(z);
  return 0;
}

/* SwiGLU -> Q8_K, per row of gu: gate = gu[0..F), up = gu[F..2F),
 *   act_k = f32(gate_k * up_k / (1 + exp(-gate_k)))   (f64, one rounding)
 * (silu(gate) * up), then the Q8_K blocks of act.  dmax as above. */
int oracle_swiglu_quantize_q8k(const float *gu, int64_t M, int64_t F, int64_t ldgu, uint8_t *out, float *dmax) {
  if (F % 256 || ldgu < 2 * F) return -1;
  const int64_t nsb = F / 256;
  float *a = (float *)malloc(sizeof(float) * (size_t)F);
  for (int64_t m = 0; m < M; ++m) {
    const float *gate = gu + m * ldgu, *up = gate + F;
    for (int64_t k = 0; k < F; ++k) {
      const double gd = (double)gate[k];
      a[k] = (float)(gd * (double)up[k] / (1.0 + exp(-gd)));
    }
    float mx = 0.0f;
    for (int64_t s = 0; s < nsb; ++s) {
      uint8_t *b = out + (m * nsb + s) * 292;
      quantize_block_q8k(a + s * 256, b);
      if (fabsf(rdf32(b)) > mx) mx = fabsf(rdf32(b));
    }
    if (dmax) dmax[m] = mx;
  }
  free(a);
  return 0;
}

/* ---- bidirectional attention ------------------------------------------- */
/* f32 -> nearest binary16 value (ties to even), as a double: the quantum is
 * 2^(e-10) for a value of exponent e >= -14 and 2^-24 below; magnitudes that
 * round to 65520 or more overflow to infinity. */
double oracle_f16_round(float x) {
  const double a = fabs((double)x);
  if (a == 0.0 || a != a) return (double)x;
  int E;
  (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1): exponent E - 1 */
  const int e = E - 1 < -14 ? -14 : E - 1;
  const double quantum = ldexp(1.0, e - 10);
  double r = rint(a / quantum) * quantum; /* a / quantum is exact; rint rounds half to even */
  if (r >= 65520.0) r = INFINITY;
  return x < 0 ? -r : r;
}

/* The pages' layer attends over the whole canvas (bidirectional, not causal)
 * after the QKV projection, on f16 tensor cores with a softmax over the keys.
 * Per head h and query i, with q, k, v rounded to f16 (the operand format):
 *   s_j = scale * sum_d q_id k_jd,  p_j = exp(s_j - max s) / sum exp(s - max s),
 *   out[i][h D + d] = sum_j p_j v_jd,
 * in f64.  qkv rows hold Q (H heads of D values), then K, then V (Hkv heads
 * each).  With grouped-query attention (Dream-7B, README milestones: "GQA"),
 * Hkv divides H and query head h reads key/value head h / (H / Hkv); Hkv = H
 * is plain multi-head attention. */
int oracle_attention(const float *qkv, int64_t L, int64_t ldqkv, int64_t H, int64_t Hkv, int64_t D, double scale,
                     double *out) {
  if (L <= 0 || H <= 0 || Hkv <= 0 || H % Hkv || D <= 0) return -1;
  const int64_t W = (H + 2 * Hkv) * D; /* Q of H heads, then K and V of Hkv heads */
  if (ldqkv < W) return -1;
  const int64_t G = H / Hkv;            /* query heads per key/value head */
  /* the operands rounded to f16 once: r[j * W + t] */
  double *r = (double *)malloc(sizeof(double) * (size_t)(L * W));
  for (int64_t j = 0; j < L; ++j)
    for (int64_t t = 0; t < W; ++t) r[j * W + t] = oracle_f16_round(qkv[j * ldqkv + t]);
  double *s = (double *)malloc(sizeof(double) * (size_t)L);
  for (int64_t h = 0; h < H; ++h) {
    const int64_t koff = H * D + (h / G) * D, voff = H * D + Hkv * D + (h / G) * D;
    for (int64_t i = 0; i < L; ++i) {
      const double *q = r + i * W + h * D;
      double mx = -INFINITY;
      for (int64_t j = 0; j < L; ++j) {
        const double *k = r + j * W + koff;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += q[d] * k[d];
        s[j] = scale * acc;
        if (s[j] > mx) mx = s[j];
      }
      double z = 0.0;
      for (int64_t j = 0; j < L; ++j) {
        s[j] = exp(s[j] - mx);
        z += s[j];
      }
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < L; ++j) acc += s[j] * r[j * W + voff + d];
        out[i * H * D + h * D + d] = acc / z;
      }
    }
  }
  free(s);
  free(r);
  return 0;
}
