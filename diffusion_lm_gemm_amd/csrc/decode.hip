// Standalone decode of Q4_K / Q6_K super-blocks into the shared form that
// both types reduce to (mojo-dllm Development plan, "Compute design", second
// bullet): unsigned bytes, an int16 scale per 16 and an f32 offset per 16,
// with the super-block factor D kept as a leading f32, so that
// w_i = D * sc[i/16] * u[i] + off[i/16].
// Record (356 B): f32 D | f32 off[16] | i16 sc[16] | u8 u[256].
// One wave per super-block; lane l writes quants 4l..4l+3.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {

template <int QT>
__global__ __launch_bounds__(256) void k_decode_qk(const uint8_t* __restrict__ w, int64_t nsb,
                                                  uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= nsb) return;
  uint8_t* o = out + s * DEC_BYTES;
  if constexpr (QT == QT_Q4K) {
    const uint8_t* b = w + s * Q4K_BYTES;  // 16-byte aligned when w is
    const uint32_t* b32 = (const uint32_t*)b;
    // quants 4l..4l+3: sub-block j = l/8, position 4(l%8) in the 32-byte run
    // 32*(j/2) of the nibble area, low nibble for even j.
    const int j = lane >> 3;
    const uint32_t v = b32[4 + 8 * (j >> 1) + (lane & 7)];
    const uint32_t u = (j & 1) ? q4k_hi_nibbles(v) : q4k_lo_nibbles(v);
    ((uint32_t*)(o + 100))[lane] = u;
    if (lane < 16) {
      uint32_t sc03, sc47, mn03, mn47;
      q4k_scales(b32[1], b32[2], b32[3], sc03, sc47, mn03, mn47);
      const int jj = lane >> 1;
      const uint32_t scb = (jj < 4) ? sc03 : sc47;
      const uint32_t mnb = (jj < 4) ? mn03 : mn47;
      const int sc = (scb >> (8 * (jj & 3))) & 63;
      const int mn = (mnb >> (8 * (jj & 3))) & 63;
      const float dmin = f16_bits_to_f32(b32[0] >> 16);
      ((int16_t*)(o + 68))[lane] = (int16_t)sc;
      ((float*)(o + 4))[lane] = -(dmin * (float)mn);
      if (lane == 0) *(float*)o = f16_bits_to_f32(b32[0]);
    }
  } else {
    const uint8_t* b = w + s * Q6K_BYTES;  // 2-byte aligned
    // quants 4l..4l+3: half h = l/32, quarter k = (l%32)/8, position
    // 4(l%8) within the quarter.
    const int h = lane >> 5, k = (lane >> 3) & 3, l = 4 * (lane & 7);
    const uint32_t ql = ld_u32_a2(b + 64 * h + 32 * (k & 1) + l);
    const uint32_t qh = ld_u32_a2(b + 128 + 32 * h + l);
    ((uint32_t*)(o + 100))[lane] = q6k_quants(ql, qh, k);
    if (lane < 16) {
      const float D = f16_bits_to_f32(*(const uint16_t*)(b + 208));
      const int sc = (int)(int8_t)b[192 + lane];
      ((int16_t*)(o + 68))[lane] = (int16_t)sc;
      ((float*)(o + 4))[lane] = -(32.0f * D * (float)sc);
      if (lane == 0) *(float*)o = D;
    }
  }
}

hipError_t launch_decode_qk(int qtype, const uint8_t* w, int64_t nsb, uint8_t* out, hipStream_t s) {
  const dim3 grid((unsigned)((nsb + 3) / 4));
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL(k_decode_qk<QT_Q4K>, grid, dim3(256), 0, s, w, nsb, out);
  else
    hipLaunchKernelGGL(k_decode_qk<QT_Q6K>, grid, dim3(256), 0, s, w, nsb, out);
  return hipGetLastError();
}

}  // namespace dllm
