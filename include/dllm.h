/*
 * libdllm -- the per-denoising-step quantized GEMM stream of a diffusion LM,
 * as hand-written HIP kernels for CDNA4 (gfx950).
 *
 * A diffusion-LM denoising step reruns the whole bidirectional transformer
 * over the whole canvas (L ~ 100..160 tokens), so every linear layer is a GEMM
 * of L per-token int8 activation rows against GGUF Q4_K / Q6_K weight rows
 * (mojo-dllm Development plan, "Compute design"; README "How it works").
 *
 * Conventions for every call:
 *  - All buffer pointers are caller-owned DEVICE pointers on the current HIP
 *    device; the library allocates nothing, keeps no state beyond its code
 *    object and never synchronizes.  `stream` is a hipStream_t (NULL = the
 *    null stream); work is only enqueued.
 *  - Sizes are int64_t.  K is always a multiple of 256 (one super-block).
 *  - Weights are row-major in GGUF order: row n (one output feature) is K/256
 *    consecutive super-blocks.  Activations are row-major per token.
 *  - Return value: 0 on success, a negative DLLM_E_* code otherwise.  Argument
 *    errors are detected on the host before anything is enqueued; the message
 *    is available from dllm_last_error() (per thread, valid until the next call
 *    on that thread).  Unsupported types fail with an explicit message and no
 *    fallback (technical specification, "GGUF" and "Error handling" sections).
 *    Device-side faults surface at the caller's next synchronization.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLLM_ABI_VERSION 11

/* qtype tags: the GGUF tensor-type ids. */
#define DLLM_Q4_K 12
#define DLLM_Q6_K 14
#define DLLM_Q8_K 15

#define DLLM_QK_K 256          /* values per super-block */
#define DLLM_Q4_K_BYTES 144    /* f16 d | f16 dmin | 12 B scales/mins | 128 B 4-bit quants */
#define DLLM_Q6_K_BYTES 210    /* 128 B low 4 bits | 64 B high 2 bits | 16 int8 scales | f16 d */
#define DLLM_Q8_K_BYTES 292    /* f32 d | 256 int8 quants | 16 int16 sums */
#define DLLM_DECODED_BYTES 356 /* f32 D | f32 off[16] | int16 sc[16] | uint8 u[256] */

#define DLLM_OK 0
#define DLLM_E_ARG (-1)         /* null pointer, bad leading dimension */
#define DLLM_E_SHAPE (-2)       /* K % 256 != 0, M <= 0, N <= 0, n_rows out of [1, M] */
#define DLLM_E_UNSUPPORTED (-3) /* qtype without a matrix kernel */
#define DLLM_E_ALIGN (-4)       /* pointer alignment not met */
#define DLLM_E_HIP (-5)         /* HIP runtime error at launch */
#define DLLM_E_WORKSPACE (-6)   /* workspace smaller than the call needs */

int dllm_abi_version(void);
const char *dllm_last_error(void);

/*
 * Q8_K activation quantization (Development plan, "Compute design", first
 * bullet: per token, int8 quants with one f32 scale per 256 values plus int
 * sums per 16 values).  Block rule (the GGUF Q8_K definition): the pivot is the
 * first value of largest magnitude in the 256-block; iscale = -127/pivot (f32,
 * correctly rounded); q = min(127, round-half-even(f32(iscale * x))); d =
 * 1/iscale; bsums[g] = sum of q[16g .. 16g+15].  An all-zero block gives d = 0,
 * q = 0, bsums = 0.  Inputs must be finite.
 *   x      f32 [M][ldx], 4-byte aligned, ldx >= K
 *   y_q8k  [M][K/256] records of 292 bytes, 4-byte aligned (written)
 *   dmax   optional f32 [M] (NULL: not written): per token, the largest |d|
 *          over its K/256 records; dllm_qgemm takes it as x_dmax
 * The output is bit-identical to the format definition.
 */
int dllm_quantize_q8k(const float *x, int64_t M, int64_t K, int64_t ldx,
                      void *y_q8k, float *dmax, void *stream);

/*
 * Fused producers of the quantized activations (Technical Specification,
 * "Transformer Execution": RMSNorm before the QKV and MLP projections, and a
 * SwiGLU MLP; Development plan, "Model facts used": RMSNorm eps 1e-5, FFN
 * 12288 SwiGLU; v0.2 goals: fused normalization).  Each writes what
 * dllm_quantize_q8k writes for the producer's output, without the f32
 * intermediate in memory.
 *
 * dllm_rmsnorm_quantize_q8k: per row of x (K values) with norm weight g [K],
 *   r = f32(1 / sqrt(sum_k x_k^2 / K + eps)), the sum of squares in f64;
 *   the records hold the codes and bsums of z = f32(x * g) (the block rule
 *   above) and d = f32(r * d_z): the records of RMSNorm(x) * g with the
 *   common factor r moved into each block's scale, so the codes are those of
 *   z exactly and only d depends on r.  K <= 16384 (DLLM_E_SHAPE otherwise);
 *   0 <= eps <= 1.  dmax as for dllm_quantize_q8k.
 *   x f32 [M][ldx] and g f32 [K], 4-byte aligned; y_q8k [M][K/256] records.
 *
 * dllm_swiglu_quantize_q8k: per row of gu (f32 [M][ldgu], ldgu >= 2F), gate
 *   = gu[m][0..F), up = gu[m][F..2F) (the layout of one GEMM over the
 *   stacked gate and up weights); the records of act = f32(gate * up /
 *   (1 + exp(-gate))) (silu(gate) * up, evaluated in f64 and rounded once);
 *   F a positive multiple of 256; y_q8k [M][F/256] records.
 */
int dllm_rmsnorm_quantize_q8k(const float *x, int64_t M, int64_t K, int64_t ldx,
                              const float *g, float eps, void *y_q8k,
                              float *dmax, void *stream);
int dllm_swiglu_quantize_q8k(const float *gu, int64_t M, int64_t F,
                             int64_t ldgu, void *y_q8k, float *dmax,
                             void *stream);

/*
 * Bidirectional attention over the canvas (Technical Specification,
 * "Transformer Execution" and "Critical difference from autoregressive
 * execution": full, not causal, attention over the diffusion region; README,
 * the GPU bullet: attention on the f16 tensor cores with a softmax over the
 * keys).  Per query head h and query i:
 *   out[i][h D + d] = sum_j softmax_j(scale * q_i . k_j) v_jd
 * over all L keys of key/value head h / (H / H_kv), with q, k, v rounded to
 * f16 (round to nearest even) and the scores, softmax and sums in f32.
 * H_kv = H is multi-head attention (LLaDA-8B); H_kv < H, dividing H, is
 * grouped-query attention (Dream-7B, README milestones: "GQA").
 *   qkv  f32 [L][ld_qkv]: per row Q (H heads of D values, head h at h*D),
 *        then K (H_kv heads), then V (H_kv heads) -- the layout of one GEMM
 *        over the stacked Q, K, V weights
 *   out  f32 [L][ld_out] (written: H*D values per row)
 *   scale  finite (1/sqrt(D) for standard attention)
 * D must be 128 and 1 <= L <= 256 (a head's keys stay in LDS): DLLM_E_SHAPE
 * otherwise; H_kv must divide H.  qkv and out 16-byte aligned,
 * ld_qkv >= (H + 2*H_kv)*D and ld_out >= H*D multiples of 4.  RoPE, if the
 * model uses it, is applied to Q and K before.
 */
int dllm_attention(const float *qkv, int64_t L, int64_t ld_qkv, int64_t H,
                   int64_t H_kv, int64_t D, float scale, float *out,
                   int64_t ld_out, void *stream);

/*
 * Decode Q4_K / Q6_K super-blocks into the shared form both types reduce to
 * (Development plan, "Compute design", second bullet: unsigned bytes, an int16
 * scale per 16 and an f32 offset per 16; the super-block factor D is kept as a
 * leading f32), so that w_i = D * sc[i/16] * u[i] + off[i/16] exactly:
 *   Q4_K: u = 4-bit quant, sc[g] = scale[g/2], off[g] = -(f32(dmin) * min[g/2])
 *   Q6_K: u = 6-bit quant (0..63), sc[g] = scale[g], off[g] = -(32 f32(d) sc[g])
 *   w    n_superblocks consecutive blocks (144 or 210 bytes), 2-byte aligned
 *   out  n_superblocks records of 356 bytes, 4-byte aligned (written)
 * Every field is exact, so the output is bit-exact.
 */
int dllm_decode_qk(int qtype, const void *w, int64_t n_superblocks,
                   void *out_decoded, void *stream);

/*
 * Quantized GEMM y[m][n] = sum_k W_hat[n][k] * X_hat[m][k] for the masked-free
 * linear layers (technical specification section 10 "Quantized Compute",
 * kernel API linear_q4k(x, weight, out); Development plan "Compute design").
 *   qtype   DLLM_Q4_K or DLLM_Q6_K
 *   w       [N][K/256] weight super-blocks, 4-byte aligned
 *   x_q8k   [M][K/256] Q8_K records (from dllm_quantize_q8k), 4-byte aligned
 *   x_dmax  optional f32 [M]: per token, the largest |d| over its records, as
 *           written by dllm_quantize_q8k (NULL: the kernel reads every
 *           record's d itself, which costs a few microseconds per call).
 *           Only Q4_K uses it, for the power-of-two range scale of its min
 *           term; the result is bit-identical with or without it.
 *   y       f32 [M][ldy], ldy >= N, 4-byte aligned (written, not accumulated)
 *   workspace / workspace_bytes   optional scratch for splitting K across
 *           work-groups; NULL/0 runs without a split.  A split needs
 *           dllm_qgemm_workspace_bytes(qtype, N, K, M) bytes, 16-byte
 *           aligned; with less the call runs without a split.  Its first
 *           64 KiB hold one arrival counter per output tile, the split's
 *           partial tiles follow: the last of a tile's work-groups to finish
 *           sums the partials in split order (in the same kernel) and sets
 *           the counter back to 0.  So the workspace must be zero-filled once
 *           before its first use, and every call leaves it ready for the next
 *           one, of any shape; calls that share a workspace must be ordered
 *           on one stream.  The result
 *           agrees with the exact dequantized product to f32 rounding either
 *           way, and is the same bits on every call.
 */
int64_t dllm_qgemm_workspace_bytes(int qtype, int64_t N, int64_t K, int64_t M);
int dllm_qgemm(int qtype, const void *w, int64_t N, int64_t K,
               const void *x_q8k, const float *x_dmax, int64_t M, float *y,
               int64_t ldy, void *workspace, int64_t workspace_bytes,
               void *stream);

/*
 * dllm_qgemm plus a bias per output feature: y[m][n] = sum_k W_hat[n][k] *
 * X_hat[m][k] + bias[n] (the Q, K and V projections of Dream-7B, README
 * milestones: "QKV bias").  bias is f32 [N], 4-byte aligned, caller-owned;
 * NULL gives exactly dllm_qgemm.  Without a K split the bias is added in the
 * GEMM's epilogue, with one in the split reduction, once either way; the
 * other arguments, the workspace rules and the errors are dllm_qgemm's.
 */
int dllm_qgemm_bias(int qtype, const void *w, int64_t N, int64_t K,
                    const void *x_q8k, const float *x_dmax, int64_t M,
                    const float *bias, float *y, int64_t ldy, void *workspace,
                    int64_t workspace_bytes, void *stream);

/*
 * Two GEMMs of one activation matrix in one launch: y_a = X_hat W_a^T (+ bias_a)
 * and y_b = X_hat W_b^T (+ bias_b), e.g. a layer's Q + K projection (Q4_K)
 * and its V projection (Q6_K), which read the same normalized hidden state
 * (Development plan, "Compute design": every linear layer multiplies the L
 * Q8_K activation rows by the layer's weight rows).  Each output is the
 * same, bit for bit, as dllm_qgemm_bias on its own with a workspace of at
 * least dllm_qgemm_workspace_bytes bytes, when this call's workspace has
 * dllm_qgemm_pair_workspace_bytes(qtype_a, N_a, qtype_b, N_b, K, M) bytes
 * (16-byte aligned; zero-filled once before first use, as dllm_qgemm's; with
 * less, or NULL, both run without a K split, as dllm_qgemm without one).
 * Where the two calls' tile plans have a grouped kernel (Q4_K tiles of 80
 * tokens with Q6_K tiles, at 129..160 tokens for the step's shapes), their
 * work-groups share one grid, so that each CU holds a tile of each; other
 * plans run as the two launches in order on the stream.
 *   qtype_*, w_*, N_*, bias_* (NULL: none), y_*, ldy_*   as for dllm_qgemm_bias
 *   K, x_q8k, x_dmax, M   shared, as for dllm_qgemm
 * y_a and y_b must not overlap each other, the workspace or the inputs.
 * Argument errors are dllm_qgemm_bias's, checked for both before anything
 * is enqueued.  dllm_qgemm_pair_workspace_bytes returns -1 for invalid
 * arguments and 0 where neither GEMM splits K.
 */
int64_t dllm_qgemm_pair_workspace_bytes(int qtype_a, int64_t N_a, int qtype_b,
                                        int64_t N_b, int64_t K, int64_t M);
int dllm_qgemm_pair(int qtype_a, const void *w_a, int64_t N_a,
                    const float *bias_a, float *y_a, int64_t ldy_a,
                    int qtype_b, const void *w_b, int64_t N_b,
                    const float *bias_b, float *y_b, int64_t ldy_b, int64_t K,
                    const void *x_q8k, const float *x_dmax, int64_t M,
                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * dllm_qgemm_bias for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same result, bit for bit, as dllm_qgemm_bias with a workspace of
 * dllm_qgemm_workspace_bytes(qtype, N, K, M) bytes, and the same plan, but
 * the K split's partial tiles and tile counters live in 24 MiB of device
 * memory that the library holds for the life of the process (one copy per
 * GPU, taken when the first call on that device finds its address).  The
 * call allocates nothing and issues no memset.  Shapes whose split would
 * need more than 24 MiB (65536 + S * M * N64 * 4 bytes, N64 = N rounded up
 * to 64) are rejected with DLLM_E_WORKSPACE; shapes that run unsplit use no
 * scratch.  The stream must belong to the current device.  Every call on a
 * GPU shares that GPU's scratch: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.
 */
int dllm_qgemm_noalloc(int qtype, const void *w, int64_t N, int64_t K,
                       const void *x_q8k, const float *x_dmax, int64_t M,
                       const float *bias, float *y, int64_t ldy,
                       void *stream);

/*
 * Masked-row LM head (Development plan, "Compute design", last bullet; README
 * "How it works", "Logits only where the sampler looks"): gather hidden rows
 * rows[0..n_rows) of h, quantize each to Q8_K, multiply by the output matrix
 * w [N][K] and write f32 logits plus the per-row argmax (greedy pick; lowest
 * index among exactly equal logits).
 *   h       f32 [M][ldh], ldh >= K
 *   rows    int32 [n_rows] device array, each in [0, M); the device code
 *           clamps an index outside [0, M) to the nearest valid row (the
 *           result for that row is then meaningless, but nothing outside h
 *           is read)
 *   logits  f32 [n_rows][ldl], ldl >= N (written)
 *   argmax  int32 [n_rows] (written)
 *   workspace  at least dllm_lmhead_workspace_bytes(qtype, N, K, n_rows) bytes,
 *           256-byte aligned (required); its contents on entry do not matter
 *           (the call writes the gathered Q8_K rows and per-wave or per-tile
 *           argmax keys there), and calls sharing one workspace must be
 *           ordered on one stream
 * n_rows may be 1..M; the kernels are tuned for n_rows <= 32 (LLaDA's block).
 */
int64_t dllm_lmhead_workspace_bytes(int qtype, int64_t N, int64_t K, int64_t n_rows);
int dllm_lmhead_masked(int qtype, const void *w, int64_t N, int64_t K,
                       const float *h, int64_t M, int64_t ldh,
                       const int32_t *rows, int64_t n_rows, float *logits,
                       int64_t ldl, int32_t *argmax, void *workspace,
                       int64_t workspace_bytes, void *stream);

/*
 * The masked-row LM head plus the confidence of the greedy pick (README
 * "How it works", "Each model's own sampler": LLaDA's low-confidence
 * remasking ranks masked positions by the softmax probability of the token
 * it would commit; Development plan, "Sampling", lists softmax, log-softmax
 * and argmax).  Everything dllm_lmhead_masked writes, and per gathered row
 *   lse       f32 [n_rows]: log(sum_n exp(logits[r][n])) over the row's N
 *             logits as written (natural log)
 *   p_argmax  f32 [n_rows]: softmax probability of argmax[r], i.e.
 *             exp(logits[r][argmax[r]] - lse[r])
 * Both are device pointers, 4-byte aligned, required.  They are computed in
 * f32 from per-wave (or per-tile) running maxima and rescaled exponential
 * sums, merged in the argmax kernel; the same workspace size applies.
 */
int dllm_lmhead_confidence(int qtype, const void *w, int64_t N, int64_t K,
                           const float *h, int64_t M, int64_t ldh,
                           const int32_t *rows, int64_t n_rows, float *logits,
                           int64_t ldl, int32_t *argmax, float *lse,
                           float *p_argmax, void *workspace,
                           int64_t workspace_bytes, void *stream);

/*
 * Test export: per-16 integer partial dots of the shared form,
 * P[m][n][sb][g] = sum_{t<16} u[n][256 sb + 16 g + t] * q[m][256 sb + 16 g + t]
 * (u: the unsigned shared-form quant, q: the Q8_K int8 quant), int32, written
 * as [M][N][K/256][16].  Computed by a separate reference kernel (v_dot4 on
 * the quants taken from the GGUF bit layout), not by the matrix kernels; the
 * matrix kernels' own integer sums are checked through
 * dllm_qgemm_superblock_sums_i32.  Meant for small shapes.
 */
int dllm_qgemm_partials_i32(int qtype, const void *w, int64_t N, int64_t K,
                            const void *x_q8k, int64_t M, int32_t *P,
                            void *stream);

/*
 * Test export: the exact int32 super-block sums the matrix kernel forms from
 * its two int8 planes (Development plan, "Compute design": the per-16 integer
 * scale form), A[m][n][sb] = (hi << shift) + lo, written as [M][N][K/256]:
 *   Q4_K: A = sum_{j<8} sc_j * sum_{t<32} u[32j + t] q[32j + t]
 *   Q6_K: A = sum_{g<16} sc_g * sum_{t<16} (u[16g + t] - 32) q[16g + t]
 * (sc the sub-block scales, u the shared-form quants, q the Q8_K quants of
 * super-block sb).  It launches dllm_qgemm's own kernel for tile
 * configuration `tile` (1..7) and K split `split` (1..K/256), in a compiled
 * form that stores each tile's integer sums where it would fold them into y;
 * the unpacking, the v_mfma_i32_16x16x64_i8 contraction and the loop are the
 * same code.  The token tile is the configuration's largest.  Meant for small
 * shapes (M * N * K/256 <= 2^31); DLLM_E_ARG for a bad tile or split.
 */
int dllm_qgemm_superblock_sums_i32(int qtype, const void *w, int64_t N,
                                   int64_t K, const void *x_q8k, int64_t M,
                                   int32_t *A, int tile, int split,
                                   void *stream);

/*
 * Test-only entry points with the kernel choice made explicit (for checking
 * every tile configuration and both LM-head paths; the product calls above
 * choose by themselves and read no environment).
 *
 * dllm_qgemm_planned: dllm_qgemm_bias with a given tile configuration and K
 *   split: tile 1..7 (the work-group shapes of the 16 x 16 tiles); split in
 *   [1, K/256] (reduced to the number of non-empty splits).  A split S > 1
 *   needs a 16-byte aligned, zero-filled workspace (dllm_qgemm's rules) of
 *   65536 + S * M * N64 * 4 bytes, N64 = N rounded up to a multiple of 64
 *   (DLLM_E_WORKSPACE otherwise).  The result agrees with dllm_qgemm to f32
 *   rounding.
 * dllm_lmhead_planned: dllm_lmhead_confidence (lse and p_argmax may both be
 *   NULL: dllm_lmhead_masked) with path 0 (choose), 1 (the streaming kernel;
 *   K <= 4096 and n_rows <= 32, DLLM_E_SHAPE otherwise) or 2 (the tiled GEMM
 *   with the argmax epilogue).
 */
int dllm_qgemm_planned(int qtype, const void *w, int64_t N, int64_t K,
                       const void *x_q8k, const float *x_dmax, int64_t M,
                       const float *bias, float *y, int64_t ldy,
                       void *workspace, int64_t workspace_bytes, int tile,
                       int split, void *stream);
int dllm_lmhead_planned(int qtype, const void *w, int64_t N, int64_t K,
                        const float *h, int64_t M, int64_t ldh,
                        const int32_t *rows, int64_t n_rows, float *logits,
                        int64_t ldl, int32_t *argmax, float *lse,
                        float *p_argmax, void *workspace,
                        int64_t workspace_bytes, int path, void *stream);

#ifdef __cplusplus
}
#endif
#endif
