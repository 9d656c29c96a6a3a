// Bidirectional attention over the canvas (the layer step between the QKV
// projection and the output projection): per head, softmax(scale Q K^T) V
// over every key, with no causal mask, on f16 operands with f32 accumulation
// (mojo-dllm Technical Specification, "Transformer Execution" and "Critical
// difference from autoregressive execution"; README, the GPU bullet: attention
// on the f16 tensor cores with a softmax over the keys).
//
// One work-group per (64 queries, query head), eight waves.  The K (row-major)
// and V^T of its key/value head (the query head itself, or with grouped-query
// attention head h / (H / Hkv)) are converted to f16 into LDS once, all keys
// (L <= 256, the canvas is about 100-160 tokens).  Wave w takes queries 16 (w & 3) ..
// +15 and one half of the 32-key chunks (w >> 2: the first ceil(C/2) chunks
// or the rest), so two waves share each SIMD and each runs half the chain:
//   S^T = K Q^T on v_mfma_f32_16x16x32_f16 (A = 16 keys from LDS, B = the
//         wave's queries in registers), 16 keys per block;
//   a softmax over the wave's keys in registers (each lane holds 4 keys of one
//         query per block; the four 16-lane groups hold the others), relative
//         to the wave's own maximum m;
//   O^T = V^T P^T on the same instruction: the score tile's own layout is the
//         B operand (a lane's 8 K slots are keys 4g..4g+3 and 16+4g..16+4g+3
//         of a 32-key chunk), and the A operand reads V^T in that key order,
//         so no data moves between the two products.
// The second half's (m, sum, O) go through LDS to its partner, which rescales
// both by exp(m_i - max(m_0, m_1)), adds them and writes the output rows with
// 16-byte stores after the division by the softmax sum.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {

namespace {

constexpr int AT_D = 128;             // head dimension
constexpr int AT_LMAX = 256;          // keys held in LDS
constexpr int AT_KS = AT_D + 8;       // halves per K row in LDS (272-byte stride: 16 rows in distinct banks)
constexpr int AT_VS = AT_LMAX + 8;    // halves per V^T row (528-byte stride: 16 rows x 8 bytes in distinct banks)
constexpr int AT_QW = 16;             // queries per wave
constexpr int AT_QG = 4;              // query groups of 16 per work-group
constexpr int AT_NW = 2 * AT_QG;      // waves per work-group: two key halves per query group
constexpr int AT_KB = AT_LMAX / 16;   // key blocks of 16

typedef _Float16 v4h __attribute__((ext_vector_type(4)));

}  // namespace

// NKB = Lp / 16 key blocks (Lp = L rounded up to whole 32-key chunks) is a
// template parameter, so every loop below is unrolled without branches and the
// compiler can overlap LDS reads, MFMAs and the softmax across key blocks.
template <int NKB>
__global__ __launch_bounds__(64 * AT_NW) void k_attention(const float* __restrict__ qkv, int64_t L, int64_t ld,
                                                        int64_t H, int64_t Hkv, float* __restrict__ out,
                                                        int64_t ldo, float scale) {
  static_assert(NKB % 2 == 0 && NKB >= 2 && NKB <= AT_KB, "whole 32-key chunks, at most AT_LMAX keys");
  __shared__ __attribute__((aligned(16))) _Float16 s_k[AT_LMAX * AT_KS];
  __shared__ __attribute__((aligned(16))) _Float16 s_vt[AT_D * AT_VS];
  constexpr int NT = 64 * AT_NW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qg = wv & (AT_QG - 1), kh = wv / AT_QG;
  const int r = lane & 15, g = lane >> 4;
  const int64_t h = blockIdx.y, hkv = h / (H / Hkv);  // query head, its key/value head
  const int Lm1 = (int)L - 1;
  const float* kbase = qkv + H * AT_D + hkv * AT_D;
  const float* vbase = qkv + (H + Hkv) * AT_D + hkv * AT_D;

  // ---- the wave's queries (B operand of S^T: dims 32c + 8g .. +7 of query
  // q0 + r), loaded first so that their latency overlaps the staging
  const int64_t qi = (int64_t)blockIdx.x * (AT_QW * AT_QG) + qg * AT_QW + r;
  float4 qraw[AT_D / 16];
  {
    const float* qp = qkv + (qi < L ? qi : L - 1) * ld + h * AT_D + 8 * g;
#pragma unroll
    for (int c = 0; c < AT_D / 32; ++c) {
      qraw[2 * c] = *(const float4*)(qp + 32 * c);
      qraw[2 * c + 1] = *(const float4*)(qp + 32 * c + 4);
    }
  }

  // ---- stage K and V^T as f16 (round to nearest even) for keys 0 .. Lp-1.
  // K items are (key, 4 dims): 32 lanes cover one 512-byte row; Lp * 32 items,
  // KI per thread.  V items are (4 keys, 4 dims), transposed in registers into
  // four 8-byte V^T row pieces; a wave's 64 items are 8 key quads (lane bits
  // 0-2) x 8 dim quads (bits 3-5), so each half-wave writes 32 distinct bank
  // pairs; Lp * 8 items (a multiple of 256, so the item bound is uniform per
  // wave).  All loads are issued before any conversion; keys at or past L load
  // a clamped in-range row and are replaced by 0.
  constexpr int KI = NKB * 16 * (AT_D / 4) / NT, NV = NKB * 16 * (AT_D / 16), VI = (NV + NT - 1) / NT;
  static_assert(KI * NT == NKB * 16 * (AT_D / 4), "K items tile the keys exactly");
  {
    float4 kv[KI], vv[VI][4];
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int e = u * NT + tid;
      kv[u] = *(const float4*)(kbase + min(e >> 5, Lm1) * ld + (e & 31) * 4);
    }
#pragma unroll
    for (int u = 0; u < VI; ++u) {
      const int e = u * NT + tid;
      if (e < NV) {
        const int T = e >> 6, jb = 8 * (T >> 2) + (e & 7), d4 = 32 * (T & 3) + 4 * ((e >> 3) & 7);
#pragma unroll
        for (int t = 0; t < 4; ++t) vv[u][t] = *(const float4*)(vbase + min(4 * jb + t, Lm1) * ld + d4);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the conversions below after every load
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int e = u * NT + tid;
      const int j = e >> 5, d4 = (e & 31) * 4;
      const float4 x = j < L ? kv[u] : float4{0.f, 0.f, 0.f, 0.f};
      *(v4h*)(s_k + j * AT_KS + d4) = v4h{(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
    }
#pragma unroll
    for (int u = 0; u < VI; ++u) {
      const int e = u * NT + tid;
      if (e < NV) {
        const int T = e >> 6, jb = 8 * (T >> 2) + (e & 7), d4 = 32 * (T & 3) + 4 * ((e >> 3) & 7);
        float4 x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = 4 * jb + t < L ? vv[u][t] : float4{0.f, 0.f, 0.f, 0.f};
        _Float16* col = s_vt + d4 * AT_VS + 4 * jb;
        *(v4h*)(col + 0 * AT_VS) = v4h{(_Float16)x[0].x, (_Float16)x[1].x, (_Float16)x[2].x, (_Float16)x[3].x};
        *(v4h*)(col + 1 * AT_VS) = v4h{(_Float16)x[0].y, (_Float16)x[1].y, (_Float16)x[2].y, (_Float16)x[3].y};
        *(v4h*)(col + 2 * AT_VS) = v4h{(_Float16)x[0].z, (_Float16)x[1].z, (_Float16)x[2].z, (_Float16)x[3].z};
        *(v4h*)(col + 3 * AT_VS) = v4h{(_Float16)x[0].w, (_Float16)x[1].w, (_Float16)x[2].w, (_Float16)x[3].w};
      }
    }
  }

  v8h qf[AT_D / 32];
  const bool qv = qi < L;
#pragma unroll
  for (int c = 0; c < AT_D / 32; ++c) {
    const float4 a = qraw[2 * c], b = qraw[2 * c + 1];
    qf[c] = qv ? v8h{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w, (_Float16)b.x, (_Float16)b.y,
                     (_Float16)b.z, (_Float16)b.w}
               : v8h{};
  }
  __syncthreads();

  // ---- the wave's 32-key chunks: the first C0 for key half 0, the rest (C0
  // or C0 - 1, possibly none) for key half 1; the count test is wave-uniform
  constexpr int NC = NKB / 2, C0 = (NC + 1) / 2;
  const int c_base = kh * C0, c_cnt = kh == 0 ? C0 : NC - C0;

  // ---- scores: lane holds S^T[32 (c_base + k2) + 16 hb + 4 g + i][query r] (keys past L: -inf)
  float sc[2 * C0][4];
#pragma unroll
  for (int k2 = 0; k2 < C0; ++k2) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int key0 = 32 * (c_base + k2) + 16 * hb;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      if (k2 < c_cnt) {
#pragma unroll
        for (int c = 0; c < AT_D / 32; ++c) {
          const v8h ka = *(const v8h*)(s_k + (key0 + r) * AT_KS + 32 * c + 8 * g);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[c], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[2 * k2 + hb][i] = (k2 < c_cnt && key0 + 4 * g + i < L) ? acc[i] * scale : -__builtin_inff();
    }
  }

  // ---- softmax over the wave's keys of query r: the lane's values, then lanes r + 16, r + 32, r + 48
  float mx = -__builtin_inff();
#pragma unroll
  for (int b = 0; b < 2 * C0; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[b][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mref = mx == -__builtin_inff() ? 0.0f : mx;  // a half with no keys: every p is 0
  float z = 0.0f;
#pragma unroll
  for (int b = 0; b < 2 * C0; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = expf(sc[b][i] - mref);
      sc[b][i] = p;
      z += p;
    }
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);

  // ---- O^T = V^T P^T over the wave's 32-key chunks, dims in 8 blocks of 16
  v4f o[AT_D / 16];
#pragma unroll
  for (int db = 0; db < AT_D / 16; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k2 = 0; k2 < C0; ++k2) {
    if (k2 < c_cnt) {
      const v8h pb = {(_Float16)sc[2 * k2][0],     (_Float16)sc[2 * k2][1],     (_Float16)sc[2 * k2][2],
                      (_Float16)sc[2 * k2][3],     (_Float16)sc[2 * k2 + 1][0], (_Float16)sc[2 * k2 + 1][1],
                      (_Float16)sc[2 * k2 + 1][2], (_Float16)sc[2 * k2 + 1][3]};
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db) {
        const _Float16* vrow = s_vt + (16 * db + r) * AT_VS + 32 * (c_base + k2);
        const v4h lo = *(const v4h*)(vrow + 4 * g);
        const v4h hi = *(const v4h*)(vrow + 16 + 4 * g);
        const v8h va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[db], 0, 0, 0);
      }
    }
  }

  // ---- merge the key halves through LDS (the K area, free once every wave is
  // past its scores): half 1 leaves (m, sum) and its 32 O values per lane in
  // the same lane slot that its partner reads
  __syncthreads();
  float* s_o = (float*)s_k;                                  // [qg][db][lane] of float4: 32 KB
  float2* s_mz = (float2*)(s_o + AT_QG * (AT_D / 16) * 64 * 4);  // [qg][lane]
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) *(v4f*)(s_o + ((qg * (AT_D / 16) + db) * 64 + lane) * 4) = o[db];
    s_mz[qg * 64 + lane] = float2{mx, z};
  }
  __syncthreads();
  if (kh == 0 && qi < L) {
    const float2 mz1 = s_mz[qg * 64 + lane];
    const float m = fmaxf(mx, mz1.x);
    const float f0 = expf(mx - m), f1 = expf(mz1.x - m);  // mz1.x = -inf with no keys: f1 = 0
    const float inv = 1.0f / (z * f0 + mz1.y * f1);
    float* op = out + qi * ldo + h * AT_D + 4 * g;
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) {
      const v4f o1 = *(const v4f*)(s_o + ((qg * (AT_D / 16) + db) * 64 + lane) * 4);
      *(v4f*)(op + 16 * db) = (o[db] * f0 + o1 * f1) * inv;
    }
  }
}

bool attention_fits(int64_t L, int64_t D) { return D == AT_D && L >= 1 && L <= AT_LMAX; }

hipError_t launch_attention(const float* qkv, int64_t L, int64_t ld, int64_t H, int64_t Hkv, float* out, int64_t ldo,
                            float scale, hipStream_t s) {
  const dim3 grid((unsigned)((L + AT_QW * AT_QG - 1) / (AT_QW * AT_QG)), (unsigned)H), block(64 * AT_NW);
  switch ((L + 31) / 32 * 2) {  // key blocks of 16 in whole 32-key chunks
    case 2: hipLaunchKernelGGL((k_attention<2>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 4: hipLaunchKernelGGL((k_attention<4>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 6: hipLaunchKernelGGL((k_attention<6>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 8: hipLaunchKernelGGL((k_attention<8>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 10: hipLaunchKernelGGL((k_attention<10>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 12: hipLaunchKernelGGL((k_attention<12>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 14: hipLaunchKernelGGL((k_attention<14>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    case 16: hipLaunchKernelGGL((k_attention<16>), grid, block, 0, s, qkv, L, ld, H, Hkv, out, ldo, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dllm
