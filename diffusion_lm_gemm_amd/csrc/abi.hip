// libdllm C ABI: host-side argument checks, launch planning and kernel
// launches.  Every check runs before anything is enqueued; messages follow
// the pages' rule that errors are explicit and actionable, with no silent
// fallback for unsupported types (technical specification, GGUF reader and
// error-handling sections).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/dllm.h"
#include "common.hpp"

#include "kernels.hpp"

using namespace dllm;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return DLLM_OK;
}

const char* qname(int qtype) {
  switch (qtype) {
    case 0: return "F32";
    case 1: return "F16";
    case 2: return "Q4_0";
    case 3: return "Q4_1";
    case 6: return "Q5_0";
    case 7: return "Q5_1";
    case 8: return "Q8_0";
    case 10: return "Q2_K";
    case 11: return "Q3_K";
    case 12: return "Q4_K";
    case 13: return "Q5_K";
    case 14: return "Q6_K";
    case 15: return "Q8_K";
    case 30: return "BF16";
    default: return "unknown";
  }
}

int check_qtype(int qtype) {
  if (qtype != DLLM_Q4_K && qtype != DLLM_Q6_K)
    return fail(DLLM_E_UNSUPPORTED,
                "unsupported weight type %s (GGUF type id %d): matrix kernels exist for Q4_K and Q6_K only",
                qname(qtype), qtype);
  return DLLM_OK;
}

bool aligned(const void* p, uintptr_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }

int check_weights(int qtype, const void* w) {
  const uintptr_t need = (qtype == DLLM_Q4_K) ? 16 : 4;
  if (!aligned(w, need))
    return fail(DLLM_E_ALIGN, "weight pointer %p must be %d-byte aligned for %s", w, (int)need, qname(qtype));
  return DLLM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DLLM_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// The GEMM kernels address weights and activations with 32-bit buffer
// offsets: each operand (plus one tile of padding rows) must stay below 2 GiB.
int check_buffer_sizes(const char* fn, int qtype, int64_t N, int64_t K, int64_t M) {
  const int64_t per = (qtype == DLLM_Q4_K) ? Q4K_BYTES : Q6K_BYTES;
  const int64_t limit = ((int64_t)1 << 31) - 1;
  if ((N + 64) * (K / 256) * per > limit)
    return fail(DLLM_E_SHAPE, "%s: weight matrix of %lld x %lld is larger than 2 GiB; split it by rows", fn,
                (long long)N, (long long)K);
  if ((M + 160) * (K / 256) * Q8K_BYTES > limit)
    return fail(DLLM_E_SHAPE, "%s: activations of %lld x %lld are larger than 2 GiB; split them by tokens", fn,
                (long long)M, (long long)K);
  return DLLM_OK;
}

// Token blocks of 16 per work-group (at most 160 tokens per work-group).
int tb_for(int64_t M) {
  const int64_t tb = cdiv(M, 16);
  return (int)(tb > 10 ? 10 : tb);
}

constexpr int64_t kCUs = 256;  // MI355X compute units

struct Plan {
  int tb;   // token blocks of 16 per work-group
  int cfg;  // tile configuration (rows per work-group: qgemm_cfg_rows(cfg))
  int64_t n_tiles, m_tiles;
  int S;    // K splits
  int sps;  // super-blocks per split
};

// Workspace of a K split: one arrival counter per output tile in a fixed
// region at the start (zero between calls, whatever the shape, so one
// workspace serves calls of different shapes), then the S partial slices
// [S][M][ldp] f32 with the row stride ldp = N rounded up to 64 (whole
// 256-byte segments per tile row; read through 32-bit offsets, so below
// 2 GiB).
constexpr int64_t kCounterBytes = 65536;
constexpr int64_t kMaxSplitTiles = kCounterBytes / 4;
int64_t split_ld(int64_t N) { return (N + 63) / 64 * 64; }

// The plan of a given configuration and K split (S is reduced to the
// number of non-empty splits; no split where the output has more tiles than
// the workspace has counters).
Plan make_plan(int cfg, int S, int64_t N, int64_t K, int64_t M) {
  const int64_t SB = K / 256;
  const int64_t sps = cdiv(SB, S);
  const int max_tb = qgemm_cfg_max_tb(cfg);
  const int tb = tb_for(M) < max_tb ? tb_for(M) : max_tb;
  const int64_t n_tiles = cdiv(N, qgemm_cfg_rows(cfg)), m_tiles = cdiv(M, (int64_t)16 * tb);
  if (n_tiles * m_tiles > kMaxSplitTiles || (int64_t)S * M * split_ld(N) * 4 >= ((int64_t)1 << 31))
    return Plan{tb, cfg, n_tiles, m_tiles, 1, (int)SB};
  return Plan{tb, cfg, n_tiles, m_tiles, (int)cdiv(SB, sps), (int)sps};
}

// Time of one super-block step of a work-group with a full token tile, per
// tile configuration, in microseconds, and its factor for Q6_K (heavier
// unpacking), fitted to measured single-GEMM times on MI355X at 148 tokens.
constexpr double kCfgStepUs[8] = {0.0, 2.610, 2.771, 2.748, 1.610, 1.871, 1.35, 2.4};
constexpr double kCfgQ6Factor[8] = {0.0, 0.873, 1.173, 1.864, 2.002, 1.039, 1.6, 1.7};

// Measured best (tile configuration, K split) for the linear layers of the
// LLaDA-8B step (d = 4096, FFN 12288; Q4_K, and Q6_K for attn_v / ffn_down)
// and of Dream-7B (d = 3584, FFN 18944) at canvases of 129..160 tokens, from
// timing every candidate on MI355X (at 148 tokens, weights streamed from HBM).
// Shapes not listed go to the cost model below.
struct Tuned {
  int qtype;
  int64_t N, K, m_lo, m_hi;
  int cfg, S;
};
constexpr Tuned kTuned[] = {
    {12, 24576, 4096, 129, 160, 7, 1},  // gate + up
    {12, 12288, 4096, 129, 160, 7, 2},  // Q + K + V
    {12, 8192, 4096, 129, 160, 6, 1},   // Q + K (V in Q6_K)
    {12, 4096, 4096, 129, 160, 6, 4},   // O
    {14, 4096, 4096, 129, 160, 6, 2},   // V (run with Q + K in one launch; alone, (5, 4) is faster)
    {12, 4096, 12288, 129, 160, 6, 4},  // down
    {14, 4096, 12288, 129, 160, 5, 8},  // down
    // Dream-7B (hidden 3584, 4 key/value heads of 128, FFN 18944)
    {12, 4608, 3584, 129, 160, 6, 1},    // Q + K + V
    {12, 4096, 3584, 129, 160, 6, 2},    // Q + K (V in Q6_K)
    {14, 512, 3584, 129, 160, 6, 14},    // V
    {12, 3584, 3584, 129, 160, 6, 2},    // O
    {12, 37888, 3584, 129, 160, 7, 1},   // gate + up
    {12, 3584, 18944, 129, 160, 7, 6},   // down
    {14, 3584, 18944, 129, 160, 2, 9},   // down
};

// Pick the tile configuration and the K split that minimise an estimate of
// the makespan: work-group rounds over the CUs times super-blocks per
// work-group times the step time, plus, for a split, the reduction at the
// end of the kernel (~1 us and ~0.54 us per MB of partials).  With no workspace, S = 1.
Plan plan_gemm(int qtype, int64_t N, int64_t K, int64_t M, bool allow_split) {
  Plan best{};
  double best_cost = 1e300;
  const int64_t SB = K / 256;
  for (const Tuned& t : kTuned) {
    if (t.qtype != qtype || t.N != N || t.K != K || M < t.m_lo || M > t.m_hi) continue;
    return make_plan(t.cfg, allow_split ? t.S : 1, N, K, M);
  }
  for (int cfg : {7, 6, 5, 4, 3, 2, 1}) {
    const int64_t smax = allow_split ? (SB < 16 ? SB : 16) : 1;
    for (int64_t S = 1; S <= smax; ++S) {
      const Plan pl = make_plan(cfg, (int)S, N, K, M);
      if (pl.S != S) continue;
      const int max_tb = qgemm_cfg_max_tb(cfg);
      // per-step time scales roughly with the tokens per work-group
      const double step_us = kCfgStepUs[cfg] * (qtype == 14 ? kCfgQ6Factor[cfg] : 1.0) *
                             (0.25 + 0.75 * (double)pl.tb / (double)max_tb);
      const int64_t wgs = pl.n_tiles * pl.m_tiles * S;
      const int64_t rounds = cdiv(wgs, kCUs);
      double cost = (double)rounds * (double)pl.sps * step_us;
      if (S > 1) cost += 1.0 + (double)S * (double)M * (double)N * 4.0 * 0.54e-6;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = pl;
      }
    }
  }
  return best;
}

int64_t split_workspace_bytes(const Plan& pl, int64_t M, int64_t N) {
  return pl.S > 1 ? kCounterBytes + (int64_t)pl.S * M * split_ld(N) * 4 : 0;
}

dim3 plan_grid(const Plan& pl) { return dim3((unsigned)pl.n_tiles, (unsigned)pl.S, (unsigned)pl.m_tiles); }

// The kernel parameters of a planned GEMM: y directly, or with a K split the
// partial slices at `slices` and one arrival counter per output tile from
// `counters` on, the reduction fused into the same kernel.
GemmParams plan_params(const Plan& pl, const void* w, int64_t N, int64_t K, const void* x_q8k, const float* x_dmax,
                       int64_t M, const float* bias, float* y, int64_t ldy, uint32_t* counters, float* slices) {
  GemmParams p{};
  p.w = (const uint8_t*)w;
  p.xq = (const uint8_t*)x_q8k;
  p.dmax = x_dmax;
  p.N = N;
  p.SB = K / 256;
  p.M = M;
  p.sps = pl.sps;
  if (pl.S == 1) {
    p.out = y;
    p.ldo = ldy;
    p.bias = bias;
  } else {
    p.out = slices;
    p.ldo = split_ld(N);
    p.split_stride = M * p.ldo;
    p.tile_cnt = counters;
    p.red_y = y;
    p.red_ldy = ldy;
    p.red_bias = bias;  // added once, by the reduction
  }
  return p;
}

// Launch a planned GEMM (a split's counters at the start of the workspace,
// its partial slices after them).
int run_plan(const char* fn, int qtype, const Plan& pl, const void* w, int64_t N, int64_t K, const void* x_q8k,
             const float* x_dmax, int64_t M, const float* bias, float* y, int64_t ldy, void* workspace,
             hipStream_t s) {
  const GemmParams p = plan_params(pl, w, N, K, x_q8k, x_dmax, M, bias, y, ldy, (uint32_t*)workspace,
                                   (float*)((uint8_t*)workspace + kCounterBytes));
  return hip_status(launch_qgemm(qtype, p, pl.tb, pl.cfg, plan_grid(pl), false, s), fn);
}

}  // namespace

extern "C" {

int dllm_abi_version(void) { return DLLM_ABI_VERSION; }

const char* dllm_last_error(void) { return g_err; }

int dllm_quantize_q8k(const float* x, int64_t M, int64_t K, int64_t ldx, void* y_q8k, float* dmax, void* stream) {
  if (!x || !y_q8k) return fail(DLLM_E_ARG, "dllm_quantize_q8k: null pointer (x=%p, y=%p)", (const void*)x, y_q8k);
  if (M <= 0 || K <= 0 || K % 256)
    return fail(DLLM_E_SHAPE, "dllm_quantize_q8k: need M > 0 and K a positive multiple of 256 (M=%lld, K=%lld)",
                (long long)M, (long long)K);
  if (ldx < K) return fail(DLLM_E_ARG, "dllm_quantize_q8k: ldx=%lld < K=%lld", (long long)ldx, (long long)K);
  if (!aligned(x, 4) || !aligned(y_q8k, 4) || !aligned(dmax, 4))
    return fail(DLLM_E_ALIGN, "dllm_quantize_q8k: x, y and dmax must be 4-byte aligned");
  if (M > 0x7fffffffLL) return fail(DLLM_E_SHAPE, "dllm_quantize_q8k: M=%lld exceeds 2^31-1", (long long)M);
  return hip_status(launch_quantize_q8k(x, ldx, nullptr, 0, M, K / 256, (uint8_t*)y_q8k, dmax, (hipStream_t)stream),
                    "dllm_quantize_q8k launch");
}

int dllm_rmsnorm_quantize_q8k(const float* x, int64_t M, int64_t K, int64_t ldx, const float* g, float eps,
                              void* y_q8k, float* dmax, void* stream) {
  const char* fn = "dllm_rmsnorm_quantize_q8k";
  if (!x || !g || !y_q8k)
    return fail(DLLM_E_ARG, "%s: null pointer (x=%p, g=%p, y=%p)", fn, (const void*)x, (const void*)g, y_q8k);
  if (M <= 0 || K <= 0 || K % 256)
    return fail(DLLM_E_SHAPE, "%s: need M > 0 and K a positive multiple of 256 (M=%lld, K=%lld)", fn, (long long)M,
                (long long)K);
  if (!rmsnorm_quantize_fits(K / 256))
    return fail(DLLM_E_SHAPE, "%s: K=%lld exceeds 16384 (the fused normalization keeps a row's block scales in LDS)",
                fn, (long long)K);
  if (ldx < K) return fail(DLLM_E_ARG, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(DLLM_E_ARG, "%s: eps=%g must be in [0, 1]", fn, (double)eps);
  if (!aligned(x, 4) || !aligned(g, 4) || !aligned(y_q8k, 4) || !aligned(dmax, 4))
    return fail(DLLM_E_ALIGN, "%s: x, g, y and dmax must be 4-byte aligned", fn);
  if (M > 0x7fffffffLL) return fail(DLLM_E_SHAPE, "%s: M=%lld exceeds 2^31-1", fn, (long long)M);
  return hip_status(launch_rmsnorm_quantize_q8k(x, ldx, M, K / 256, g, eps, (uint8_t*)y_q8k, dmax, (hipStream_t)stream),
                    "dllm_rmsnorm_quantize_q8k launch");
}

int dllm_swiglu_quantize_q8k(const float* gu, int64_t M, int64_t F, int64_t ldgu, void* y_q8k, float* dmax,
                             void* stream) {
  const char* fn = "dllm_swiglu_quantize_q8k";
  if (!gu || !y_q8k) return fail(DLLM_E_ARG, "%s: null pointer (gu=%p, y=%p)", fn, (const void*)gu, y_q8k);
  if (M <= 0 || F <= 0 || F % 256)
    return fail(DLLM_E_SHAPE, "%s: need M > 0 and F a positive multiple of 256 (M=%lld, F=%lld)", fn, (long long)M,
                (long long)F);
  if (ldgu < 2 * F) return fail(DLLM_E_ARG, "%s: ldgu=%lld < 2F=%lld", fn, (long long)ldgu, (long long)(2 * F));
  if (!aligned(gu, 4) || !aligned(y_q8k, 4) || !aligned(dmax, 4))
    return fail(DLLM_E_ALIGN, "%s: gu, y and dmax must be 4-byte aligned", fn);
  if (M > 0x7fffffffLL) return fail(DLLM_E_SHAPE, "%s: M=%lld exceeds 2^31-1", fn, (long long)M);
  return hip_status(launch_swiglu_quantize_q8k(gu, ldgu, M, F / 256, (uint8_t*)y_q8k, dmax, (hipStream_t)stream),
                    "dllm_swiglu_quantize_q8k launch");
}

int dllm_attention(const float* qkv, int64_t L, int64_t ld_qkv, int64_t H, int64_t H_kv, int64_t D, float scale,
                   float* out, int64_t ld_out, void* stream) {
  const char* fn = "dllm_attention";
  if (!qkv || !out) return fail(DLLM_E_ARG, "%s: null pointer (qkv=%p, out=%p)", fn, (const void*)qkv, (void*)out);
  if (H <= 0 || L <= 0 || H_kv <= 0 || H % H_kv)
    return fail(DLLM_E_SHAPE, "%s: need L > 0, H > 0 and H_kv > 0 dividing H (L=%lld, H=%lld, H_kv=%lld)", fn,
                (long long)L, (long long)H, (long long)H_kv);
  if (!attention_fits(L, D))
    return fail(DLLM_E_SHAPE, "%s: head dimension %lld and L=%lld: this kernel takes D = 128 and 1 <= L <= 256 "
                "(every key of a head held in LDS)", fn, (long long)D, (long long)L);
  if (ld_qkv < (H + 2 * H_kv) * D)
    return fail(DLLM_E_ARG, "%s: ld_qkv=%lld < (H + 2*H_kv)*D=%lld", fn, (long long)ld_qkv,
                (long long)((H + 2 * H_kv) * D));
  if (ld_out < H * D) return fail(DLLM_E_ARG, "%s: ld_out=%lld < H*D=%lld", fn, (long long)ld_out, (long long)(H * D));
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return fail(DLLM_E_ARG, "%s: scale must be finite", fn);
  if (!aligned(qkv, 16) || !aligned(out, 16) || ld_qkv % 4 || ld_out % 4)
    return fail(DLLM_E_ALIGN, "%s: qkv and out must be 16-byte aligned with row strides a multiple of 4", fn);
  if (H > 65535) return fail(DLLM_E_SHAPE, "%s: H=%lld exceeds 65535", fn, (long long)H);
  return hip_status(launch_attention(qkv, L, ld_qkv, H, H_kv, out, ld_out, scale, (hipStream_t)stream),
                    "dllm_attention launch");
}

int dllm_decode_qk(int qtype, const void* w, int64_t n_superblocks, void* out, void* stream) {
  int rc = check_qtype(qtype);
  if (rc) return rc;
  if (!w || !out) return fail(DLLM_E_ARG, "dllm_decode_qk: null pointer (w=%p, out=%p)", w, out);
  if (n_superblocks <= 0) return fail(DLLM_E_SHAPE, "dllm_decode_qk: n_superblocks=%lld must be > 0", (long long)n_superblocks);
  if ((rc = check_weights(qtype, w))) return rc;
  if (!aligned(out, 4)) return fail(DLLM_E_ALIGN, "dllm_decode_qk: out must be 4-byte aligned");
  return hip_status(launch_decode_qk(qtype, (const uint8_t*)w, n_superblocks, (uint8_t*)out, (hipStream_t)stream),
                    "dllm_decode_qk launch");
}

int64_t dllm_qgemm_workspace_bytes(int qtype, int64_t N, int64_t K, int64_t M) {
  if (check_qtype(qtype) || N <= 0 || M <= 0 || K <= 0 || K % 256) return -1;
  return split_workspace_bytes(plan_gemm(qtype, N, K, M, true), M, N);
}

static int check_gemm_args(const char* fn, int qtype, const void* w, int64_t N, int64_t K, const void* xq, int64_t M) {
  int rc = check_qtype(qtype);
  if (rc) return rc;
  if (!w || !xq) return fail(DLLM_E_ARG, "%s: null pointer (w=%p, x_q8k=%p)", fn, w, xq);
  if (N <= 0 || M <= 0 || K <= 0 || K % 256)
    return fail(DLLM_E_SHAPE, "%s: need N > 0, M > 0 and K a positive multiple of 256 (N=%lld, K=%lld, M=%lld)", fn,
                (long long)N, (long long)K, (long long)M);
  if (N > 0x7fffffffLL) return fail(DLLM_E_SHAPE, "%s: N=%lld exceeds 2^31-1", fn, (long long)N);
  if ((rc = check_weights(qtype, w))) return rc;
  if (!aligned(xq, 4)) return fail(DLLM_E_ALIGN, "%s: x_q8k must be 4-byte aligned", fn);
  if ((rc = check_buffer_sizes(fn, qtype, N, K, M))) return rc;
  return DLLM_OK;
}

// dllm_qgemm, and with a bias dllm_qgemm_bias.
static int qgemm_impl(const char* fn, int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k,
                      const float* x_dmax, int64_t M, const float* bias, float* y, int64_t ldy, void* workspace,
                      int64_t workspace_bytes, void* stream) {
  int rc = check_gemm_args(fn, qtype, w, N, K, x_q8k, M);
  if (rc) return rc;
  if (!y) return fail(DLLM_E_ARG, "%s: null output pointer", fn);
  if (ldy < N) return fail(DLLM_E_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (!aligned(y, 4) || !aligned(x_dmax, 4) || !aligned(bias, 4))
    return fail(DLLM_E_ALIGN, "%s: y, x_dmax and bias must be 4-byte aligned", fn);
  Plan pl = plan_gemm(qtype, N, K, M, true);
  const int64_t need = split_workspace_bytes(pl, M, N);
  if (pl.S > 1 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    pl = plan_gemm(qtype, N, K, M, false);  // no usable workspace: whole K range per work-group
  return run_plan(fn, qtype, pl, w, N, K, x_q8k, x_dmax, M, bias, y, ldy, workspace, (hipStream_t)stream);
}

int dllm_qgemm(int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k, const float* x_dmax, int64_t M,
               float* y, int64_t ldy, void* workspace, int64_t workspace_bytes, void* stream) {
  return qgemm_impl("dllm_qgemm", qtype, w, N, K, x_q8k, x_dmax, M, nullptr, y, ldy, workspace, workspace_bytes,
                    stream);
}

int dllm_qgemm_bias(int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k, const float* x_dmax,
                    int64_t M, const float* bias, float* y, int64_t ldy, void* workspace, int64_t workspace_bytes,
                    void* stream) {
  return qgemm_impl("dllm_qgemm_bias", qtype, w, N, K, x_q8k, x_dmax, M, bias, y, ldy, workspace, workspace_bytes,
                    stream);
}

// ---- dllm_qgemm_pair: two GEMMs of one activation matrix, one launch -----

namespace {
// Workspace of a pair: the counters (A's tiles first, then B's), A's slices,
// B's slices.  Without a split on either side, none.
struct PairPlan {
  Plan a, b;
  int64_t cnt_b;           // B's first counter
  int64_t slices_a_bytes;  // bytes of A's slices (0 unsplit)
  int64_t need;            // workspace bytes
};
int64_t split_slice_bytes(const Plan& pl, int64_t M, int64_t N) {
  return pl.S > 1 ? (int64_t)pl.S * M * split_ld(N) * 4 : 0;
}
PairPlan plan_pair(int qa, int64_t Na, int qb, int64_t Nb, int64_t K, int64_t M, bool allow_split) {
  PairPlan pp{};
  pp.a = plan_gemm(qa, Na, K, M, allow_split);
  pp.b = plan_gemm(qb, Nb, K, M, allow_split);
  pp.cnt_b = pp.a.S > 1 ? pp.a.n_tiles * pp.a.m_tiles : 0;
  // both splits' counters must fit the counter region; B's shifts after A's
  if (pp.b.S > 1 && pp.cnt_b + pp.b.n_tiles * pp.b.m_tiles > kMaxSplitTiles) pp.cnt_b = 0;
  pp.slices_a_bytes = split_slice_bytes(pp.a, M, Na);
  const int64_t sb = split_slice_bytes(pp.b, M, Nb);
  pp.need = (pp.slices_a_bytes + sb) > 0 ? kCounterBytes + pp.slices_a_bytes + sb : 0;
  return pp;
}
}  // namespace

int64_t dllm_qgemm_pair_workspace_bytes(int qtype_a, int64_t N_a, int qtype_b, int64_t N_b, int64_t K, int64_t M) {
  if (check_qtype(qtype_a) || check_qtype(qtype_b) || N_a <= 0 || N_b <= 0 || M <= 0 || K <= 0 || K % 256) return -1;
  return plan_pair(qtype_a, N_a, qtype_b, N_b, K, M, true).need;
}

int dllm_qgemm_pair(int qtype_a, const void* w_a, int64_t N_a, const float* bias_a, float* y_a, int64_t ldy_a,
                    int qtype_b, const void* w_b, int64_t N_b, const float* bias_b, float* y_b, int64_t ldy_b,
                    int64_t K, const void* x_q8k, const float* x_dmax, int64_t M, void* workspace,
                    int64_t workspace_bytes, void* stream) {
  const char* fn = "dllm_qgemm_pair";
  int rc = check_gemm_args(fn, qtype_a, w_a, N_a, K, x_q8k, M);
  if (rc) return rc;
  if ((rc = check_gemm_args(fn, qtype_b, w_b, N_b, K, x_q8k, M))) return rc;
  if (!y_a || !y_b) return fail(DLLM_E_ARG, "%s: null output pointer (y_a=%p, y_b=%p)", fn, (void*)y_a, (void*)y_b);
  if (ldy_a < N_a || ldy_b < N_b)
    return fail(DLLM_E_ARG, "%s: need ldy_a >= N_a and ldy_b >= N_b (ldy_a=%lld, N_a=%lld, ldy_b=%lld, N_b=%lld)", fn,
                (long long)ldy_a, (long long)N_a, (long long)ldy_b, (long long)N_b);
  if (!aligned(y_a, 4) || !aligned(y_b, 4) || !aligned(x_dmax, 4) || !aligned(bias_a, 4) || !aligned(bias_b, 4))
    return fail(DLLM_E_ALIGN, "%s: y_a, y_b, x_dmax and the biases must be 4-byte aligned", fn);
  PairPlan pp = plan_pair(qtype_a, N_a, qtype_b, N_b, K, M, true);
  if (pp.need > 0 && (!workspace || workspace_bytes < pp.need || !aligned(workspace, 16)))
    pp = plan_pair(qtype_a, N_a, qtype_b, N_b, K, M, false);  // no usable workspace: no split on either side
  // (a plan without a split uses neither counters nor slices)
  uint8_t* const ws = pp.need > 0 ? (uint8_t*)workspace : nullptr;
  uint32_t* const cnt_a = ws ? (uint32_t*)ws : nullptr;
  uint32_t* const cnt_b = ws ? (uint32_t*)ws + pp.cnt_b : nullptr;
  float* const slices_a = ws ? (float*)(ws + kCounterBytes) : nullptr;
  float* const slices_b = ws ? (float*)(ws + kCounterBytes + pp.slices_a_bytes) : nullptr;
  const GemmParams pa = plan_params(pp.a, w_a, N_a, K, x_q8k, x_dmax, M, bias_a, y_a, ldy_a, cnt_a, slices_a);
  const GemmParams pb = plan_params(pp.b, w_b, N_b, K, x_q8k, x_dmax, M, bias_b, y_b, ldy_b, cnt_b, slices_b);
  const hipStream_t s = (hipStream_t)stream;
  const bool counters_apart = pp.b.S == 1 || pp.a.S == 1 || pp.cnt_b > 0;
  const int64_t wgs = pp.a.n_tiles * pp.a.S * pp.a.m_tiles + pp.b.n_tiles * pp.b.S * pp.b.m_tiles;
  if (counters_apart && wgs + 16 < 0x7fffffffLL &&
      qgemm_pair_fits(qtype_a, pp.a.cfg, pp.a.tb, qtype_b, pp.b.cfg, pp.b.tb))
    return hip_status(launch_qgemm_pair(qtype_a, pa, pp.a.tb, pp.a.cfg, plan_grid(pp.a), qtype_b, pb, pp.b.tb,
                                        pp.b.cfg, plan_grid(pp.b), s),
                      fn);
  // no grouped kernel for these two plans: the two launches in order on the
  // stream (the second may then reuse the first one's counters)
  rc = hip_status(launch_qgemm(qtype_a, pa, pp.a.tb, pp.a.cfg, plan_grid(pp.a), false, s), fn);
  if (rc) return rc;
  return hip_status(launch_qgemm(qtype_b, pb, pp.b.tb, pp.b.cfg, plan_grid(pp.b), false, s), fn);
}

// ---- dllm_qgemm_noalloc: the K split in memory the library holds --------

namespace {
// The split's tile counters and partial slices (the workspace layout of
// dllm_qgemm) in a file-scope device array: zero when the code object is
// loaded, one copy per GPU, held until the process ends.  Every call leaves
// the counter region zero again.  Host code only ever uses the address that
// hipGetSymbolAddress returns for the current device, never the array's name.
constexpr int64_t kScratchBytes = (int64_t)24 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, set on the first call there

int scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DLLM_E_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DLLM_E_HIP, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DLLM_E_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DLLM_OK;
}
}  // namespace

int dllm_qgemm_noalloc(int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k, const float* x_dmax,
                       int64_t M, const float* bias, float* y, int64_t ldy, void* stream) {
  const char* fn = "dllm_qgemm_noalloc";
  int rc = check_gemm_args(fn, qtype, w, N, K, x_q8k, M);
  if (rc) return rc;
  if (!y) return fail(DLLM_E_ARG, "%s: null output pointer", fn);
  if (ldy < N) return fail(DLLM_E_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (!aligned(y, 4) || !aligned(x_dmax, 4) || !aligned(bias, 4))
    return fail(DLLM_E_ALIGN, "%s: y, x_dmax and bias must be 4-byte aligned", fn);
  const Plan pl = plan_gemm(qtype, N, K, M, true);  // dllm_qgemm's plan with a large enough workspace
  const int64_t need = split_workspace_bytes(pl, M, N);
  if (need > kScratchBytes)
    return fail(DLLM_E_WORKSPACE,
                "%s: the K split of this shape (N=%lld, K=%lld, M=%lld) needs %lld bytes of scratch, more than the "
                "%lld the library holds; call dllm_qgemm_bias with a workspace instead",
                fn, (long long)N, (long long)K, (long long)M, (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  if (pl.S > 1 && (rc = scratch_for_current_device(fn, &ws))) return rc;
  return run_plan(fn, qtype, pl, w, N, K, x_q8k, x_dmax, M, bias, y, ldy, ws, (hipStream_t)stream);
}

// Key slots per gathered row: one per 64-row tile (tiled path) or one per
// wave (streaming path), whichever is more.
static int64_t lmhead_slots(int64_t N) {
  return cdiv(N, 64) > lmhead_stream_waves() ? cdiv(N, 64) : lmhead_stream_waves();
}

// Workspace: the gathered Q8_K rows, then per slot and row an argmax key (u64)
// and softmax statistics (two f32).
int64_t dllm_lmhead_workspace_bytes(int qtype, int64_t N, int64_t K, int64_t n_rows) {
  if (check_qtype(qtype) || N <= 0 || K <= 0 || K % 256 || n_rows <= 0) return -1;
  return align256(n_rows * (K / 256) * Q8K_BYTES) + align256(lmhead_slots(N) * n_rows * 8) +
         lmhead_slots(N) * n_rows * 8;
}

// dllm_lmhead_masked, and with lse / p_max (both or neither) dllm_lmhead_confidence.
// path: 0 chooses (the streaming kernel where it applies), 1 forces the
// streaming kernel, 2 the tiled GEMM with the argmax epilogue.
static int lmhead_impl(const char* fn, int qtype, const void* w, int64_t N, int64_t K, const float* h, int64_t M,
                       int64_t ldh, const int32_t* rows, int64_t n_rows, float* logits, int64_t ldl,
                       int32_t* argmax, float* lse, float* p_max, void* workspace, int64_t workspace_bytes,
                       int path, void* stream) {
  int rc = check_qtype(qtype);
  if (rc) return rc;
  if (!w || !h || !rows || !logits || !argmax || !workspace)
    return fail(DLLM_E_ARG,
                "%s: null pointer (w=%p, h=%p, rows=%p, logits=%p, argmax=%p, workspace=%p)", fn, w,
                (const void*)h, (const void*)rows, (void*)logits, (void*)argmax, workspace);
  if (N <= 0 || M <= 0 || K <= 0 || K % 256)
    return fail(DLLM_E_SHAPE, "%s: need N > 0, M > 0, K a positive multiple of 256 (N=%lld, K=%lld, M=%lld)", fn,
                (long long)N, (long long)K, (long long)M);
  if (n_rows < 1 || n_rows > M)
    return fail(DLLM_E_SHAPE, "%s: n_rows=%lld must be in [1, M=%lld]", fn, (long long)n_rows, (long long)M);
  if (N > 0x7fffffffLL) return fail(DLLM_E_SHAPE, "%s: N=%lld exceeds 2^31-1", fn, (long long)N);
  if ((rc = check_buffer_sizes(fn, qtype, N, K, n_rows))) return rc;
  if (ldh < K) return fail(DLLM_E_ARG, "%s: ldh=%lld < K=%lld", fn, (long long)ldh, (long long)K);
  if (ldl < N) return fail(DLLM_E_ARG, "%s: ldl=%lld < N=%lld", fn, (long long)ldl, (long long)N);
  if ((rc = check_weights(qtype, w))) return rc;
  if (!aligned(h, 4) || !aligned(logits, 4) || !aligned(rows, 4) || !aligned(argmax, 4))
    return fail(DLLM_E_ALIGN, "%s: h, rows, logits and argmax must be 4-byte aligned", fn);
  if (!aligned(workspace, 256)) return fail(DLLM_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if ((lse == nullptr) != (p_max == nullptr))
    return fail(DLLM_E_ARG, "%s: lse and p_argmax are both given or both null (lse=%p, p_argmax=%p)", fn, (void*)lse,
                (void*)p_max);
  if (!aligned(lse, 4) || !aligned(p_max, 4)) return fail(DLLM_E_ALIGN, "%s: lse and p_argmax must be 4-byte aligned", fn);
  const int64_t need = dllm_lmhead_workspace_bytes(qtype, N, K, n_rows);
  if (workspace_bytes < need)
    return fail(DLLM_E_WORKSPACE, "%s: workspace of %lld bytes, need %lld", fn, (long long)workspace_bytes,
                (long long)need);
  if (path < 0 || path > 2) return fail(DLLM_E_ARG, "%s: path=%d must be 0, 1 or 2", fn, path);
  if (path == 1 && !lmhead_stream_fits(K, n_rows))
    return fail(DLLM_E_SHAPE, "%s: the streaming LM head takes K <= 4096 and n_rows <= 32 (K=%lld, n_rows=%lld)", fn,
                (long long)K, (long long)n_rows);
  hipStream_t s = (hipStream_t)stream;
  const int64_t SB = K / 256;
  uint8_t* xq = (uint8_t*)workspace;
  uint64_t* keys = (uint64_t*)((uint8_t*)workspace + align256(n_rows * SB * Q8K_BYTES));
  float2* stats = lse ? (float2*)((uint8_t*)keys + align256(lmhead_slots(N) * n_rows * 8)) : nullptr;
  if ((rc = hip_status(launch_quantize_q8k(h, ldh, rows, M, n_rows, SB, xq, nullptr, s), "lm head gather/quantize launch")))
    return rc;
  if (path != 2 && lmhead_stream_fits(K, n_rows)) {
    LmParams lp;
    lp.w = (const uint8_t*)w;
    lp.xq = xq;
    lp.logits = logits;
    lp.keys = keys;
    lp.stats = stats;
    lp.N = N;
    lp.SB = SB;
    lp.M = n_rows;
    lp.ldl = ldl;
    if ((rc = hip_status(launch_lmhead_stream(qtype, lp, s), "lm head stream launch"))) return rc;
    return hip_status(launch_argmax_finalize(keys, stats, lmhead_stream_slots(N), n_rows, argmax, lse, p_max, s),
                      "lm head argmax launch");
  }
  GemmParams p{};
  p.w = (const uint8_t*)w;
  p.xq = xq;
  p.dmax = nullptr;
  p.out = logits;
  p.keys = keys;
  p.stats = stats;
  p.bias = nullptr;
  p.N = N;
  p.SB = SB;
  p.M = n_rows;
  p.ldo = ldl;
  p.split_stride = 0;
  p.sps = (int)SB;
  const int tb = tb_for(n_rows);
  const int64_t n_tiles = cdiv(N, 64);  // 4 waves, 64 rows per work-group
  const dim3 grid((unsigned)n_tiles, 1, (unsigned)cdiv(n_rows, 16 * tb));
  if ((rc = hip_status(launch_qgemm(qtype, p, tb, 5, grid, true, s), "lm head gemm launch"))) return rc;
  return hip_status(launch_argmax_finalize(keys, stats, n_tiles, n_rows, argmax, lse, p_max, s), "lm head argmax launch");
}

int dllm_lmhead_masked(int qtype, const void* w, int64_t N, int64_t K, const float* h, int64_t M, int64_t ldh,
                       const int32_t* rows, int64_t n_rows, float* logits, int64_t ldl, int32_t* argmax,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  return lmhead_impl("dllm_lmhead_masked", qtype, w, N, K, h, M, ldh, rows, n_rows, logits, ldl, argmax, nullptr,
                     nullptr, workspace, workspace_bytes, 0, stream);
}

int dllm_lmhead_confidence(int qtype, const void* w, int64_t N, int64_t K, const float* h, int64_t M, int64_t ldh,
                           const int32_t* rows, int64_t n_rows, float* logits, int64_t ldl, int32_t* argmax,
                           float* lse, float* p_argmax, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!lse || !p_argmax)
    return fail(DLLM_E_ARG, "dllm_lmhead_confidence: null pointer (lse=%p, p_argmax=%p)", (void*)lse, (void*)p_argmax);
  return lmhead_impl("dllm_lmhead_confidence", qtype, w, N, K, h, M, ldh, rows, n_rows, logits, ldl, argmax, lse,
                     p_argmax, workspace, workspace_bytes, 0, stream);
}

int dllm_qgemm_partials_i32(int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k, int64_t M, int32_t* P,
                            void* stream) {
  int rc = check_gemm_args("dllm_qgemm_partials_i32", qtype, w, N, K, x_q8k, M);
  if (rc) return rc;
  if (!P) return fail(DLLM_E_ARG, "dllm_qgemm_partials_i32: null output pointer");
  if (!aligned(P, 4)) return fail(DLLM_E_ALIGN, "dllm_qgemm_partials_i32: P must be 4-byte aligned");
  if (M * N * (K / 256) * 16 > ((int64_t)1 << 40))
    return fail(DLLM_E_SHAPE, "dllm_qgemm_partials_i32: output too large for a test export");
  return hip_status(launch_partials(qtype, (const uint8_t*)w, N, K / 256, (const uint8_t*)x_q8k, M, P,
                                    (hipStream_t)stream),
                    "dllm_qgemm_partials_i32 launch");
}

// ---- test-only entry points ------------------------------------------------

int dllm_qgemm_planned(int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k, const float* x_dmax,
                       int64_t M, const float* bias, float* y, int64_t ldy, void* workspace, int64_t workspace_bytes,
                       int tile, int split, void* stream) {
  const char* fn = "dllm_qgemm_planned";
  int rc = check_gemm_args(fn, qtype, w, N, K, x_q8k, M);
  if (rc) return rc;
  if (!y) return fail(DLLM_E_ARG, "%s: null output pointer", fn);
  if (ldy < N) return fail(DLLM_E_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (!aligned(y, 4) || !aligned(x_dmax, 4) || !aligned(bias, 4))
    return fail(DLLM_E_ALIGN, "%s: y, x_dmax and bias must be 4-byte aligned", fn);
  if (tile < 1 || tile > 7) return fail(DLLM_E_ARG, "%s: tile=%d must be 1..7", fn, tile);
  if (split < 1 || split > K / 256) return fail(DLLM_E_ARG, "%s: split=%d must be in [1, K/256]", fn, split);
  const Plan pl = make_plan(tile, split, N, K, M);
  if (pl.S > 1) {
    const int64_t need = split_workspace_bytes(pl, M, N);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
      return fail(DLLM_E_WORKSPACE, "%s: split %d needs a 16-byte aligned workspace of %lld bytes", fn, pl.S,
                  (long long)need);
  }
  return run_plan(fn, qtype, pl, w, N, K, x_q8k, x_dmax, M, bias, y, ldy, workspace, (hipStream_t)stream);
}

int dllm_lmhead_planned(int qtype, const void* w, int64_t N, int64_t K, const float* h, int64_t M, int64_t ldh,
                        const int32_t* rows, int64_t n_rows, float* logits, int64_t ldl, int32_t* argmax, float* lse,
                        float* p_argmax, void* workspace, int64_t workspace_bytes, int path, void* stream) {
  return lmhead_impl("dllm_lmhead_planned", qtype, w, N, K, h, M, ldh, rows, n_rows, logits, ldl, argmax, lse,
                     p_argmax, workspace, workspace_bytes, path, stream);
}

int dllm_qgemm_superblock_sums_i32(int qtype, const void* w, int64_t N, int64_t K, const void* x_q8k, int64_t M,
                                   int32_t* A, int tile, int split, void* stream) {
  const char* fn = "dllm_qgemm_superblock_sums_i32";
  int rc = check_gemm_args(fn, qtype, w, N, K, x_q8k, M);
  if (rc) return rc;
  if (!A) return fail(DLLM_E_ARG, "%s: null output pointer", fn);
  if (!aligned(A, 4)) return fail(DLLM_E_ALIGN, "%s: A must be 4-byte aligned", fn);
  if (tile < 1 || tile > 7) return fail(DLLM_E_ARG, "%s: tile=%d must be 1..7", fn, tile);
  if (split < 1 || split > K / 256) return fail(DLLM_E_ARG, "%s: split=%d must be in [1, K/256]", fn, split);
  if (M * N * (K / 256) > ((int64_t)1 << 31)) return fail(DLLM_E_SHAPE, "%s: output too large for a test export", fn);
  // the test form runs the configuration's largest token tile
  Plan pl = make_plan(tile, split, N, K, M);
  pl.tb = qgemm_cfg_max_tb(tile);
  pl.m_tiles = cdiv(M, (int64_t)16 * pl.tb);
  GemmParams p{};
  p.w = (const uint8_t*)w;
  p.xq = (const uint8_t*)x_q8k;
  p.dmax = nullptr;
  p.out = (float*)A;
  p.keys = nullptr;
  p.stats = nullptr;
  p.bias = nullptr;
  p.N = N;
  p.SB = K / 256;
  p.M = M;
  p.ldo = N;
  p.split_stride = 0;
  p.sps = pl.sps;
  const dim3 grid((unsigned)pl.n_tiles, (unsigned)pl.S, (unsigned)pl.m_tiles);
  return hip_status(launch_qgemm_sums(qtype, p, tile, grid, (hipStream_t)stream), fn);
}

}  // extern "C"
