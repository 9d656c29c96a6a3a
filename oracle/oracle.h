/* CPU oracle API -- test infrastructure only (see oracle.c). */
#ifndef DLLM_ORACLE_H
#define DLLM_ORACLE_H
#include <stdint.h>

#define ORACLE_Q4_K 12
#define ORACLE_Q6_K 14

double oracle_f16_to_f64(uint16_t h);
void oracle_q4k_fields(const uint8_t *b, double *d, double *dmin, int sc[8],
                       int mn[8], int u[256]);
void oracle_q6k_fields(const uint8_t *b, double *d, int sc[16], int q[256]);
int oracle_decode_rows(int qtype, const uint8_t *w, int64_t N, int64_t K,
                       double *out);
int oracle_decode_shared(int qtype, const uint8_t *w, int64_t nsb, uint8_t *out);
int oracle_quantize_q8k(const float *x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t *out);
int oracle_dequant_q8k(const uint8_t *xq, int64_t M, int64_t K, double *out);
int oracle_gemm(int qtype, const uint8_t *w, int64_t N, int64_t K,
                const uint8_t *xq, int64_t M, double *y, int nthreads);
int oracle_gemm_sample(int qtype, const uint8_t *w, int64_t N, int64_t K,
                       const uint8_t *xq, int64_t M, const int64_t *mi,
                       const int64_t *ni, int64_t count, double *out);
int oracle_partials(int qtype, const uint8_t *w, int64_t N, int64_t K,
                    const uint8_t *xq, int64_t M, int32_t *P);
int oracle_lmhead(int qtype, const uint8_t *w, int64_t N, int64_t K,
                  const float *h, int64_t M, int64_t ldh, const int32_t *rows,
                  int64_t n_rows, double *logits, int32_t *argmax, int nthreads);
int oracle_softmax_stats(const double *logits, int64_t n_rows, int64_t N,
                         double *lse, double *p_argmax);
int oracle_rmsnorm_quantize_q8k(const float *x, int64_t M, int64_t K, int64_t ldx,
                                const float *g, float eps, uint8_t *out, float *dmax);
int oracle_swiglu_quantize_q8k(const float *gu, int64_t M, int64_t F, int64_t ldgu,
                               uint8_t *out, float *dmax);
double oracle_f16_round(float x);
int oracle_attention(const float *qkv, int64_t L, int64_t ldqkv, int64_t H,
                     int64_t Hkv, int64_t D, double scale, double *out);
#endif
