// Bidirectional attention over the canvas (the layer step between the QKV
// projection and the output projection): per head, softmax(scale Q K^T) V
// over every key, with no causal mask, on f16 operands with f32 accumulation
// (mojo-dllm Technical Specification, "Transformer Execution" and "Critical
// difference from autoregressive execution"; README, the GPU bullet: attention
// on the f16 tensor cores with a softmax over the keys).
//
// One work-group per (64 queries, head).  The head's K (row-major) and V^T are
// converted to f16 into LDS once, all keys (L <= 256, the canvas is about
// 100-160 tokens).  Each wave takes 16 queries:
//   S^T = K Q^T on v_mfma_f32_16x16x32_f16 (A = 16 keys from LDS, B = the
//         wave's queries in registers), 16 keys per block;
//   an exact softmax over all keys in registers (each lane holds 4 keys of one
//         query per block; the four 16-lane groups hold the others);
//   O^T = V^T P^T on the same instruction: the score tile's own layout is the
//         B operand (a lane's 8 K slots are keys 4g..4g+3 and 16+4g..16+4g+3
//         of a 32-key chunk), and the A operand reads V^T in that key order,
//         so no data moves between the two products.
// The output rows are written with 16-byte stores after the division by the
// softmax sum.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {

namespace {

constexpr int AT_D = 128;             // head dimension
constexpr int AT_LMAX = 256;          // keys held in LDS
constexpr int AT_KS = AT_D + 8;       // halves per K row in LDS (272-byte stride: 16 rows in distinct banks)
constexpr int AT_VS = AT_LMAX + 8;    // halves per V^T row (528-byte stride)
constexpr int AT_QW = 16;             // queries per wave
constexpr int AT_NW = 4;              // waves per work-group
constexpr int AT_KB = AT_LMAX / 16;   // key blocks of 16

typedef _Float16 v4h __attribute__((ext_vector_type(4)));

}  // namespace

__global__ __launch_bounds__(64 * AT_NW) void k_attention(const float* __restrict__ qkv, int64_t L, int64_t ld,
                                                        int64_t H, float* __restrict__ out, int64_t ldo,
                                                        float scale) {
  __shared__ __attribute__((aligned(16))) _Float16 s_k[AT_LMAX * AT_KS];
  __shared__ __attribute__((aligned(16))) _Float16 s_vt[AT_D * AT_VS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t h = blockIdx.y;
  const int Lp = (int)((L + 31) / 32) * 32;  // keys padded to whole 32-key chunks (zero K and V)
  const float* kbase = qkv + H * AT_D + h * AT_D;
  const float* vbase = qkv + 2 * H * AT_D + h * AT_D;

  // ---- stage K and V^T as f16 (round to nearest even)
  for (int e = tid; e < Lp * (AT_D / 4); e += 64 * AT_NW) {
    const int j = e / (AT_D / 4), d4 = (e - j * (AT_D / 4)) * 4;
    float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
    if (j < L) {
      kv = *(const float4*)(kbase + j * ld + d4);
      vv = *(const float4*)(vbase + j * ld + d4);
    }
    const v4h k4 = {(_Float16)kv.x, (_Float16)kv.y, (_Float16)kv.z, (_Float16)kv.w};
    *(v4h*)(s_k + j * AT_KS + d4) = k4;
    s_vt[(d4 + 0) * AT_VS + j] = (_Float16)vv.x;
    s_vt[(d4 + 1) * AT_VS + j] = (_Float16)vv.y;
    s_vt[(d4 + 2) * AT_VS + j] = (_Float16)vv.z;
    s_vt[(d4 + 3) * AT_VS + j] = (_Float16)vv.w;
  }

  // ---- the wave's queries: B operand of S^T, dims 32c + 8g .. +7 of query q0 + r
  const int64_t qi = (int64_t)blockIdx.x * (AT_QW * AT_NW) + wv * AT_QW + r;
  v8h qf[AT_D / 32];
#pragma unroll
  for (int c = 0; c < AT_D / 32; ++c) {
    float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (qi < L) {
      const float* qp = qkv + qi * ld + h * AT_D + 32 * c + 8 * g;
      a = *(const float4*)qp;
      b = *(const float4*)(qp + 4);
    }
    qf[c] = v8h{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
  }
  __syncthreads();

  // ---- scores: lane holds S^T[16 b + 4 g + i][query r] (keys past L: -inf)
  const int nkb = Lp / 16;
  float sc[AT_KB][4];
#pragma unroll
  for (int b = 0; b < AT_KB; ++b) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (b < nkb) {
#pragma unroll
      for (int c = 0; c < AT_D / 32; ++c) {
        const v8h ka = *(const v8h*)(s_k + (16 * b + r) * AT_KS + 32 * c + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[c], acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[b][i] = (16 * b + 4 * g + i < L) ? acc[i] * scale : -__builtin_inff();
  }

  // ---- softmax over the keys of query r: the lane's values, then lanes r + 16, r + 32, r + 48
  float mx = -__builtin_inff();
#pragma unroll
  for (int b = 0; b < AT_KB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[b][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float z = 0.0f;
#pragma unroll
  for (int b = 0; b < AT_KB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = expf(sc[b][i] - mx);
      sc[b][i] = p;
      z += p;
    }
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);

  // ---- O^T = V^T P^T over 32-key chunks, dims in 8 blocks of 16
  v4f o[AT_D / 16];
#pragma unroll
  for (int db = 0; db < AT_D / 16; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k2 = 0; k2 < AT_KB / 2; ++k2) {
    if (2 * k2 < nkb) {
      const v8h pb = {(_Float16)sc[2 * k2][0],     (_Float16)sc[2 * k2][1],     (_Float16)sc[2 * k2][2],
                      (_Float16)sc[2 * k2][3],     (_Float16)sc[2 * k2 + 1][0], (_Float16)sc[2 * k2 + 1][1],
                      (_Float16)sc[2 * k2 + 1][2], (_Float16)sc[2 * k2 + 1][3]};
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db) {
        const _Float16* vrow = s_vt + (16 * db + r) * AT_VS + 32 * k2;
        const v4h lo = *(const v4h*)(vrow + 4 * g);
        const v4h hi = *(const v4h*)(vrow + 16 + 4 * g);
        const v8h va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[db], 0, 0, 0);
      }
    }
  }

  // ---- lane holds O^T[16 db + 4 g + i][query r]: four consecutive dims
  if (qi < L) {
    const float inv = 1.0f / z;
    float* op = out + qi * ldo + h * AT_D + 4 * g;
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) *(v4f*)(op + 16 * db) = o[db] * inv;
  }
}

bool attention_fits(int64_t L, int64_t D) { return D == AT_D && L >= 1 && L <= AT_LMAX; }

hipError_t launch_attention(const float* qkv, int64_t L, int64_t ld, int64_t H, float* out, int64_t ldo, float scale,
                            hipStream_t s) {
  const dim3 grid((unsigned)((L + AT_QW * AT_NW - 1) / (AT_QW * AT_NW)), (unsigned)H);
  hipLaunchKernelGGL(k_attention, grid, dim3(64 * AT_NW), 0, s, qkv, L, ld, H, out, ldo, scale);
  return hipGetLastError();
}

}  // namespace dllm
