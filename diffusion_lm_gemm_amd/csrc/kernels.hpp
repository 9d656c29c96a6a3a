// Host-side launch entry points of the libdllm kernels (one per .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

struct GemmParams {
  const uint8_t* w;
  const uint8_t* xq;
  const float* dmax;     // per token, the largest |d| of its blocks, or null
  float* out;            // y (no split) or split partials
  uint64_t* keys;        // argmax keys [n_tiles][M] (LM head) or null
  float2* stats;         // with keys: softmax statistics (m, s) [n_tiles][M], or null
  const float* bias;     // f32 [N] added to every output row (no split only), or null
  int64_t N, SB, M;
  int64_t ldo;           // leading dimension of out
  int64_t split_stride;  // floats between split slices of out
  int sps;               // super-blocks per split
  // K split with its reduction fused (tile_cnt not null): out holds the
  // split slices; the last of a tile's split work-groups to finish sums them
  // in split order, adds red_bias (or nothing), writes red_y, and resets the
  // tile's arrival counter tile_cnt[blockIdx.z * gridDim.x + blockIdx.x] to 0
  uint32_t* tile_cnt;
  float* red_y;
  int64_t red_ldy;
  const float* red_bias;
};

// Streaming LM head: at most 32 gathered Q8_K rows (xq, [M][SB] records)
// against all N weight rows; keys[wave * M + m] get each wave's best key.
struct LmParams {
  const uint8_t* w;
  const uint8_t* xq;
  float* logits;
  uint64_t* keys;
  float2* stats;  // softmax statistics (m, s) [wave][M], or null
  int64_t N, SB, M;
  int64_t ldl;
};

// rows (or null): output row m quantizes x row rows[m], clamped into [0, n_src).
hipError_t launch_quantize_q8k(const float* x, int64_t ldx, const int32_t* rows, int64_t n_src, int64_t M, int64_t SB,
                               uint8_t* y, float* dmax, hipStream_t s);
// Fused producers (RMSNorm -> Q8_K with K <= 16384, SwiGLU -> Q8_K; see quantize.hip).
bool rmsnorm_quantize_fits(int64_t SB);
hipError_t launch_rmsnorm_quantize_q8k(const float* x, int64_t ldx, int64_t M, int64_t SB, const float* g, float eps,
                                       uint8_t* y, float* dmax, hipStream_t s);
hipError_t launch_swiglu_quantize_q8k(const float* gu, int64_t ldgu, int64_t M, int64_t SB, uint8_t* y, float* dmax,
                                      hipStream_t s);
// Bidirectional attention (attention.hip): head dimension 128, 1 <= L <= 256;
// H query heads over Hkv key/value heads (Hkv divides H).
bool attention_fits(int64_t L, int64_t D);
hipError_t launch_attention(const float* qkv, int64_t L, int64_t ld, int64_t H, int64_t Hkv, float* out, int64_t ldo,
                            float scale, hipStream_t s);
hipError_t launch_decode_qk(int qtype, const uint8_t* w, int64_t nsb, uint8_t* out, hipStream_t s);
// cfg: tile configuration (1: 64 rows, 4 waves x 16; 2: 128 rows, 8 waves x 16;
// 3: 256 rows, 8 waves x 32, up to 80 tokens; 4: 128 rows, 4 waves x 32, up
// to 80 tokens; 5: 64 rows, 4 waves x 16, one activation stage, two
// work-groups per CU; 6: 64 rows, 4 waves x 16, up to 80 tokens, two
// work-groups per CU; 7: 192 rows, 12 waves x 16, up to 80 tokens).  argmax
// forces cfg 5.
int qgemm_cfg_rows(int cfg);
int qgemm_cfg_max_tb(int cfg);
hipError_t launch_qgemm(int qtype, const GemmParams& p, int tb, int cfg, dim3 grid, bool argmax, hipStream_t s);
// Two planned GEMMs of one activation matrix in one launch, their
// work-groups interleaved over one grid (each tile computes what it computes
// in its own launch); qgemm_pair_fits says which pairs of (type, cfg, token
// tile) have a grouped kernel.
bool qgemm_pair_fits(int qtype_a, int cfg_a, int tb_a, int qtype_b, int cfg_b, int tb_b);
hipError_t launch_qgemm_pair(int qtype_a, const GemmParams& pa, int tb_a, int cfg_a, dim3 grid_a, int qtype_b,
                             const GemmParams& pb, int tb_b, int cfg_b, dim3 grid_b, hipStream_t s);
// The same kernels in their test form: the exact int32 super-block sums
// A[m][n][sb] go to p.out instead of y; token tile qgemm_cfg_max_tb(cfg).
hipError_t launch_qgemm_sums(int qtype, const GemmParams& p, int cfg, dim3 grid, hipStream_t s);
bool lmhead_stream_fits(int64_t K, int64_t n_rows);
int lmhead_stream_waves();             // the most waves (key slots per row) it uses
int64_t lmhead_stream_slots(int64_t N);  // the waves it uses for N rows
hipError_t launch_lmhead_stream(int qtype, const LmParams& p, hipStream_t s);
// stats != nullptr: also lse[m] = log-sum-exp and p_max[m] = softmax probability
// of the argmax, from the per-tile (m, s) statistics.
hipError_t launch_argmax_finalize(const uint64_t* keys, const float2* stats, int64_t n_tiles, int64_t M,
                                  int32_t* argmax, float* lse, float* p_max, hipStream_t s);
hipError_t launch_partials(int qtype, const uint8_t* w, int64_t N, int64_t SB, const uint8_t* xq, int64_t M,
                           int32_t* P, hipStream_t s);

}  // namespace dllm
