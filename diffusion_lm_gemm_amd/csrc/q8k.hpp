// The Q8_K block rule for one wave (the activation quantization of the
// quantized GEMM: int8 quants, one f32 scale per 256 values, int sums per
// 16; mojo-dllm Development plan, "Compute design", first bullet), shared by
// the quantizer kernel and the GEMM's producer work-groups, which must write
// the same bytes.  Reductions use DPP moves inside 16-lane rows and lane
// reads across rows, so a block costs no LDS round trips.
#pragma once

#include "common.hpp"

namespace dllm {

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

// The Q8_K block rule on one 256-value block held by a wave as v[0..3] =
// values 4 lane .. 4 lane + 3: the pivot is the first value of largest
// magnitude, iscale = -127/pivot, q = min(127, round-half-even(f32(iscale*x))),
// d = 1/iscale, bsums = sums of 16; every step in f32 with correctly rounded
// division and no contraction.  Returns the lane's four quants packed as
// bytes, the sum of its quad's 16 quants (every lane of the quad holds it)
// and d (0 for an all-zero block, whose quants are 0).
struct Q8Block {
  uint32_t packed;
  uint32_t bsum;
  float d;
};

__device__ __forceinline__ Q8Block q8k_block(const float (&v)[4], int lane) {
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
  Q8Block b;
  b.packed = (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8) | ((uint32_t)(q[2] & 255) << 16) |
             ((uint32_t)(q[3] & 255) << 24);
  // sum of 16 = the four lanes of a quad
  uint32_t sm = (uint32_t)(q[0] + q[1] + q[2] + q[3]);
  sm += dpp<DPP_QUAD_SWAP1>(sm);
  sm += dpp<DPP_QUAD_SWAP2>(sm);
  b.bsum = sm;
  b.d = zero ? 0.0f : 1.0f / iscale;
  return b;
}

// Four consecutive f32 values; vec when p is 16-byte aligned.
__device__ __forceinline__ void load4_f32(const float* p, bool vec, float (&v)[4]) {
  if (vec) {
    const float4 t = *(const float4*)p;
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i];
  }
}

}  // namespace dllm
