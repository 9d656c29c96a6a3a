// Q8_K activation quantization: one wave per 256-value block.
//
// Per token, int8 quants with one f32 scale per 256 values plus int sums per
// 16 values (mojo-dllm Development plan, "Compute design", first bullet).  The
// block rule is the GGUF Q8_K definition: pivot = first value of largest
// magnitude, iscale = -127/pivot, q = min(127, round-half-even(f32(iscale*x))),
// d = 1/iscale, bsums = sums of 16.  Every step is done in f32 with correctly
// rounded division and no contraction, so the bytes equal the definition's.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {

// Lane l owns values 4l..4l+3 of the block.  rows != nullptr gathers token m
// from row rows[m] of x (masked-row LM head).
__global__ __launch_bounds__(256) void k_quantize_q8k(const float* __restrict__ x, int64_t ldx,
                                                     const int32_t* __restrict__ rows,
                                                     int64_t M, int64_t SB,
                                                     uint8_t* __restrict__ y) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= M * SB) return;
  const int64_t m = blk / SB, sb = blk - m * SB;
  const int64_t src_row = rows ? (int64_t)rows[m] : m;
  const float* xb = x + src_row * ldx + sb * QK + 4 * lane;
  float v[4];
  if ((((uintptr_t)xb) & 15) == 0) {
    const float4 t = *(const float4*)xb;
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    for (int i = 0; i < 4; ++i) v[i] = xb[i];
  }
  // First index of the largest magnitude: strict '>' in ascending order
  // inside the lane, then (larger magnitude, else smaller index) across lanes.
  float amax = 0.0f;
  int aidx = 0x7fffffff;
  for (int i = 0; i < 4; ++i) {
    const float a = __builtin_fabsf(v[i]);
    if (a > amax) { amax = a; aidx = 4 * lane + i; }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float oa = __shfl_xor(amax, off);
    const int oi = __shfl_xor(aidx, off);
    if (oa > amax || (oa == amax && oi < aidx)) { amax = oa; aidx = oi; }
  }
  uint8_t* out = y + blk * Q8K_BYTES;
  if (amax == 0.0f) {
    ((uint32_t*)(out + 4))[lane] = 0u;
    if (lane < 8) ((uint32_t*)(out + 260))[lane] = 0u;
    if (lane == 0) *(float*)out = 0.0f;
    return;
  }
  // The pivot value itself (signed), from the lane that holds it.
  const int src_lane = aidx >> 2, src_i = aidx & 3;
  float pv = (src_i == 0) ? v[0] : (src_i == 1) ? v[1] : (src_i == 2) ? v[2] : v[3];
  const float pivot = __shfl(pv, src_lane);
  const float iscale = -127.0f / pivot;
  int q[4];
  for (int i = 0; i < 4; ++i) {
    const float p = iscale * v[i];
    int t = (int)__builtin_rintf(p);
    q[i] = t > 127 ? 127 : t;
  }
  const uint32_t packed = (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8) |
                          ((uint32_t)(q[2] & 255) << 16) | ((uint32_t)(q[3] & 255) << 24);
  ((uint32_t*)(out + 4))[lane] = packed;
  // Sum of 16 = four consecutive lanes.
  int s = q[0] + q[1] + q[2] + q[3];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if ((lane & 3) == 0) ((int16_t*)(out + 260))[lane >> 2] = (int16_t)s;
  if (lane == 0) *(float*)out = 1.0f / iscale;
}

hipError_t launch_quantize_q8k(const float* x, int64_t ldx, const int32_t* rows, int64_t M, int64_t SB, uint8_t* y,
                               hipStream_t s) {
  const int64_t blocks = M * SB;
  hipLaunchKernelGGL(k_quantize_q8k, dim3((unsigned)((blocks + 3) / 4)), dim3(256), 0, s, x, ldx, rows, M, SB, y);
  return hipGetLastError();
}

}  // namespace dllm
