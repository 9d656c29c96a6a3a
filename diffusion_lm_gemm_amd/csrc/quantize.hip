// Q8_K activation quantization: one work-group per token row.
//
// Per token, int8 quants with one f32 scale per 256 values plus int sums per
// 16 values (mojo-dllm Development plan, "Compute design", first bullet).  The
// block rule is the GGUF Q8_K definition: pivot = first value of largest
// magnitude, iscale = -127/pivot, q = min(127, round-half-even(f32(iscale*x))),
// d = 1/iscale, bsums = sums of 16.  Every step is done in f32 with correctly
// rounded division and no contraction, so the bytes equal the definition's.
//
// Each of the QW waves of a work-group takes the row's super-blocks w,
// w + QW, ..., QU of them at a time with their loads in flight together and
// no branch between them, so their reductions interleave.  The block maximum
// is reduced with DPP row moves inside each 16-lane row and lane reads across
// rows, so a block costs no LDS round trips.  The row's largest |d| is also
// reduced (optional output): the matrix kernel takes its power-of-two range
// scale from it instead of scanning every block's d.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {

namespace {

constexpr int QW = 16;  // waves per work-group (one token row)

// DPP controls (quad permutes and row mirrors move data inside 4- and
// 16-lane groups without touching LDS).
constexpr int DPP_QUAD_SWAP1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int DPP_QUAD_SWAP2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <-> 15 - i within a row of 16
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <-> 7 - i within a half row

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Largest of a non-negative f32 (as its bits, which order like the values)
// over the wave; the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t v) {
  v = max(v, dpp<DPP_QUAD_SWAP1>(v));
  v = max(v, dpp<DPP_QUAD_SWAP2>(v));
  v = max(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dpp<DPP_ROW_MIRROR>(v));  // every lane holds its row's maximum
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Quantize one 256-value block held as v[0..3] = values 4 lane .. 4 lane + 3
// into the 292-byte record at `out` (written only if `store`); returns |d|.
__device__ __forceinline__ float quantize_block(const float (&v)[4], uint8_t* out, int lane, bool store) {
#pragma clang fp contract(off)
  float a[4];
  float lm = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_fabsf(v[i]);
    lm = fmaxf(lm, a[i]);
  }
  const float amax = __builtin_bit_cast(float, wave_max_bits(__builtin_bit_cast(uint32_t, lm)));
  // an all-zero block gives d = 0 and zero quants (selects, not a branch)
  const bool zero = (amax == 0.0f);
  // the pivot: the first value of largest magnitude, i.e. the lowest lane
  // holding the maximum and, inside it, the lowest position
  const int first = (a[0] == amax) ? 0 : (a[1] == amax) ? 1 : (a[2] == amax) ? 2 : (a[3] == amax) ? 3 : 4;
  const uint64_t holders = __ballot(first < 4);
  const int src_lane = __builtin_ctzll(holders);
  const float pv = (first == 0) ? v[0] : (first == 1) ? v[1] : (first == 2) ? v[2] : v[3];
  const float pivot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), src_lane));
  const float iscale = -127.0f / (zero ? 1.0f : pivot);
  int q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = iscale * v[i];
    const int t = (int)__builtin_rintf(p);
    q[i] = zero ? 0 : (t > 127 ? 127 : t);
  }
  const uint32_t packed = (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8) |
                          ((uint32_t)(q[2] & 255) << 16) | ((uint32_t)(q[3] & 255) << 24);
  // sum of 16 = the four lanes of a quad
  uint32_t s = (uint32_t)(q[0] + q[1] + q[2] + q[3]);
  s += dpp<DPP_QUAD_SWAP1>(s);
  s += dpp<DPP_QUAD_SWAP2>(s);
  const float d = zero ? 0.0f : 1.0f / iscale;
  if (store) {
    ((uint32_t*)(out + 4))[lane] = packed;
    if ((lane & 3) == 0) ((int16_t*)(out + 260))[lane >> 2] = (int16_t)(int32_t)s;
    if (lane == 0) *(float*)out = d;
  }
  return store ? __builtin_fabsf(d) : 0.0f;
}

}  // namespace

// rows != nullptr gathers token m from row rows[m] of x (masked-row LM head);
// dmax != nullptr receives each row's largest |d|.  QU = blocks per wave in
// flight: a block index past the row loads the row's last block again and
// stores nothing.
template <int QU>
__global__ __launch_bounds__(64 * QW) void k_quantize_q8k(const float* __restrict__ x, int64_t ldx,
                                                     const int32_t* __restrict__ rows, int64_t SB,
                                                     uint8_t* __restrict__ y, float* __restrict__ dmax) {
  __shared__ float s_wmax[QW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t m = blockIdx.x;
  const int64_t src_row = rows ? (int64_t)rows[m] : m;
  const float* xrow = x + src_row * ldx;
  // every lane's 16 bytes are aligned exactly when the row start is
  const bool vec = ((((uintptr_t)xrow) & 15) == 0);
  float wmax = 0.0f;
  for (int64_t sb0 = wv; sb0 < SB; sb0 += QW * QU) {
    float v[QU][4];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t sb = sb0 + QW * u < SB ? sb0 + QW * u : SB - 1;
      const float* xb = xrow + sb * QK + 4 * lane;
      if (vec) {
        const float4 t = *(const float4*)xb;
        v[u][0] = t.x; v[u][1] = t.y; v[u][2] = t.z; v[u][3] = t.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[u][i] = xb[i];
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t sb = sb0 + QW * u;
      wmax = fmaxf(wmax, quantize_block(v[u], y + (m * SB + sb) * Q8K_BYTES, lane, sb < SB));
    }
  }
  if (dmax) {
    if (lane == 0) s_wmax[wv] = wmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float r = s_wmax[0];
#pragma unroll
      for (int k = 1; k < QW; ++k) r = fmaxf(r, s_wmax[k]);
      dmax[m] = r;
    }
  }
}

hipError_t launch_quantize_q8k(const float* x, int64_t ldx, const int32_t* rows, int64_t M, int64_t SB, uint8_t* y,
                               float* dmax, hipStream_t s) {
  // enough blocks in flight per wave to cover rows of up to 64 blocks in one
  // round (K = 4096: one per wave; K = 12288: three)
  const int64_t per_wave = (SB + QW - 1) / QW;
  const dim3 grid((unsigned)M), block(64 * QW);
  if (per_wave <= 1)
    hipLaunchKernelGGL(k_quantize_q8k<1>, grid, block, 0, s, x, ldx, rows, SB, y, dmax);
  else if (per_wave == 2)
    hipLaunchKernelGGL(k_quantize_q8k<2>, grid, block, 0, s, x, ldx, rows, SB, y, dmax);
  else if (per_wave == 3)
    hipLaunchKernelGGL(k_quantize_q8k<3>, grid, block, 0, s, x, ldx, rows, SB, y, dmax);
  else
    hipLaunchKernelGGL(k_quantize_q8k<4>, grid, block, 0, s, x, ldx, rows, SB, y, dmax);
  return hipGetLastError();
}

}  // namespace dllm
