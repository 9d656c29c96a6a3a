// Weight-side building blocks shared by the GEMM and LM-head kernels: the K
// order of the MFMA fragments, raw super-block loads, and the unpacking of
// Q4_K / Q6_K blocks into two exact int8 planes (GGUF block layouts; the
// mojo-dllm Development plan, "Compute design", names the types and the
// per-16 scale form).
#pragma once

#include "common.hpp"

namespace dllm {

// LDS holds each token's 256 activation bytes in natural K order as sixteen
// 16-byte units, unit u of token tok stored at unit slot u ^ (tok & 15): the
// 16-byte B-fragment reads of 16 consecutive tokens then fall in 16 distinct
// slots (no bank conflicts), and the rows stay dense, so buffer-to-LDS loads
// (which write 16 bytes per lane to consecutive addresses) can fill them by
// choosing which global unit each lane fetches.
constexpr int ACT_ROW = 256;

template <int QT>
struct QTr;
template <>
struct QTr<QT_Q4K> {
  static constexpr int BYTES = Q4K_BYTES;
  static constexpr int SHIFT = 3;
  static constexpr int RAW = 12;  // dwords of raw block data per lane
};
template <>
struct QTr<QT_Q6K> {
  static constexpr int BYTES = Q6K_BYTES;
  static constexpr int SHIFT = 7;
  static constexpr int RAW = 21;
};

__device__ __forceinline__ uint32_t pkmul(uint32_t a, uint32_t b) {
  return as_u32(as_u16x2(a) * as_u16x2(b));
}

// K order of the MFMA fragments.  For K chunk c (0..3) of a super-block,
// lane group g4 (lanes 16 g4 .. 16 g4 + 15) holds 16 consecutive K values,
// activation unit act_unit<QT>(c, g4) (bytes 16 u .. 16 u + 15 of the block).
// Chunks are chosen so that each lane unpacks them from bytes it loads itself,
// with a nibble choice that is the same for every lane of a chunk:
//   Q4_K: chunk c = (half h = c >> 1, nibble n = c & 1): the n-nibbles of
//         quant bytes 64 h + 16 g4 .. + 15, i.e. sub-block 4h + 2(g4 >> 1) + n,
//         positions 16 (g4 & 1) .. + 15.
//   Q6_K: chunk c = (half h = c >> 1, nibble n = c & 1): low-bit bytes
//         64 h + 16 g4 .. + 15 (nibble n) with high-bit bytes
//         32 h + 16 (g4 & 1) .. + 15, i.e. quarter k = 2n + (g4 >> 1) of half h,
//         positions 16 (g4 & 1) .. + 15.
template <int QT>
__device__ __forceinline__ int act_unit(int c, int g4) {
  if constexpr (QT == QT_Q4K) return 8 * (c >> 1) + 4 * (g4 >> 1) + 2 * (c & 1) + (g4 & 1);
  else return 8 * (c >> 1) + 4 * (c & 1) + g4;
}

// Raw (packed) bytes of the lane's part of one weight super-block at byte
// offset `off` of the weight buffer.  Reads past the end of the buffer (rows
// beyond N) return zeros, so padded rows contribute nothing.
template <int QT>
__device__ __forceinline__ void load_raw(rsrc_t wr, uint32_t off, int g4, uint32_t (&raw)[QTr<QT>::RAW]) {
  if constexpr (QT == QT_Q4K) {
    // header (d | dmin, 12 scale/min bytes), then quant bytes 16 g4 .. and
    // 64 + 16 g4 .. of the 128-byte quant area.  Blocks are 144 bytes, so
    // every piece is 16-byte aligned.
    const v4u hdr = buf_ld128(wr, off);
    const v4u q0 = buf_ld128(wr, off + 16 + 16 * g4);
    const v4u q1 = buf_ld128(wr, off + 16 + 64 + 16 * g4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw[i] = hdr[i];
      raw[4 + i] = q0[i];
      raw[8 + i] = q1[i];
    }
  } else {
    // Blocks are 210 bytes, so a block starts at a dword boundary or two
    // bytes past one; the 16-byte loads take the fields at their byte
    // offsets (buffer loads need no dword alignment).  Fields: low-bit bytes
    // 64h + 16 g4 (h = 0, 1), high-bit bytes 128 + 32h + 16 (g4 & 1), the 16
    // scales at 192, and the f16 d at 208 (a 16-bit load: a dword there would
    // reach past the end of the buffer for the last block, and the buffer's
    // range check would zero all of it).
    const v4u f[5] = {buf_ld128(wr, off + 16 * g4), buf_ld128(wr, off + 64 + 16 * g4),
                      buf_ld128(wr, off + 128 + 16 * (g4 & 1)), buf_ld128(wr, off + 160 + 16 * (g4 & 1)),
                      buf_ld128(wr, off + 192)};
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[4 * k + i] = f[k][i];
    raw[20] = buf_ld16(wr, off + 208);
  }
}

// Dword-aligned form of the raw loads, for streams bound by memory latency
// (where a 16-byte load two bytes past a dword boundary costs more than the
// byte alignment afterwards): Q6_K fields as the five dwords that cover each,
// brought to the load_raw layout by align_raw once the data has arrived.
template <int QT>
struct QTw {
  static constexpr int RAW = (QT == QT_Q6K) ? 26 : QTr<QT>::RAW;
};

template <int QT>
__device__ __forceinline__ void load_raw_dw(rsrc_t wr, uint32_t off, int g4, uint32_t (&w)[QTw<QT>::RAW]) {
  if constexpr (QT == QT_Q4K) {
    load_raw<QT>(wr, off, g4, w);
  } else {
    const uint32_t a = off & ~3u;
    const uint32_t fo[5] = {a + 16 * g4, a + 64 + 16 * g4, a + 128 + 16 * (g4 & 1), a + 160 + 16 * (g4 & 1), a + 192};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const v4u v = buf_ld128(wr, fo[k]);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[5 * k + i] = v[i];
      w[5 * k + 4] = buf_ld32(wr, fo[k] + 16);
    }
    w[25] = buf_ld16(wr, off + 208);
  }
}

// load_raw_dw data of a block at byte offset `off` -> the load_raw layout.
template <int QT>
__device__ __forceinline__ void align_raw(const uint32_t (&w)[QTw<QT>::RAW], uint32_t off,
                                          uint32_t (&raw)[QTr<QT>::RAW]) {
  if constexpr (QT == QT_Q4K) {
#pragma unroll
    for (int i = 0; i < QTr<QT>::RAW; ++i) raw[i] = w[i];
  } else {
    const uint32_t soff = off & 3u;
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[4 * k + i] = __builtin_amdgcn_alignbyte(w[5 * k + i + 1], w[5 * k + i], soff);
    raw[20] = w[25];
  }
}

// Q6_K: four quants (bytes, 0..63) with one signed scale s -> the two int8
// planes of s*(q-32).  In 16-bit lanes 2s*q - 64s = 2 s (q-32) = 256 hi + 2 lo,
// so the high byte is hi and the low byte is 2 lo.
__device__ __forceinline__ void q6_planes(uint32_t q, uint32_t s2, uint32_t c64, uint32_t& lo, uint32_t& hi) {
  const uint32_t e = __builtin_amdgcn_perm(0u, q, 0x0c020c00u);  // q0, q2 in u16 lanes
  const uint32_t o = __builtin_amdgcn_perm(0u, q, 0x0c030c01u);  // q1, q3
  const uint32_t we = as_u32(as_u16x2(e) * as_u16x2(s2) + as_u16x2(c64));
  const uint32_t wo = as_u32(as_u16x2(o) * as_u16x2(s2) + as_u16x2(c64));
  hi = __builtin_amdgcn_perm(wo, we, 0x07030501u);
  lo = __builtin_amdgcn_perm(wo, we, 0x06020400u) >> 1;
}

// Q6_K: the four 6-bit quants of one dword for K chunk nibble N: the N-nibbles
// of the low-bit bytes ql with, at bits 4..5, the 2-bit field of quarter
// k = 2N + (g4 >> 1) of the high-bit bytes qh (bits 2k..2k+1 of each byte).
// The field is shifted into place whole-dword and masked with the nibbles in
// one and-or; what a shift carries in from a neighbouring byte is masked off.
template <int N>
__device__ __forceinline__ uint32_t q6_quants(uint32_t ql, uint32_t qh, int g4) {
  const int k2 = 2 * (g4 >> 1);
  if constexpr (N == 0) return ((qh << (4 - k2)) & 0x30303030u) | (ql & 0x0F0F0F0Fu);
  else return ((qh >> k2) & 0x30303030u) | ((ql >> 4) & 0x0F0F0F0Fu);
}

// Q6_K: the signed scale of K chunk (h, n) for this lane's row and the u16x2
// splats of 2s and -64s (q6_planes' factor and addend).
__device__ __forceinline__ void q6_scale(uint32_t scd, int g4, uint32_t& s2, uint32_t& c64) {
  const int sc = (int)(int8_t)(scd >> (8 * g4));
  s2 = __builtin_amdgcn_perm(0u, (uint32_t)(2 * sc), 0x01000100u);
  c64 = __builtin_amdgcn_perm(0u, (uint32_t)(-64 * sc), 0x01000100u);
}

// Unpack raw bytes into the two int8 planes of the four 16x64 A fragments
// (K order of act_unit) and return the super-block factor d.
template <int QT>
__device__ __forceinline__ float unpack(const uint32_t (&raw)[QTr<QT>::RAW], int g4, v4i (&alo)[4], v4i (&ahi)[4]) {
  if constexpr (QT == QT_Q4K) {
    uint32_t sc03, sc47, mn03, mn47;
    q4k_scales(raw[1], raw[2], raw[3], sc03, sc47, mn03, mn47);
    const int jb0 = 2 * (g4 >> 1);  // sub-block byte of chunk (h, 0); chunk (h, 1) is the next one
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int h = c >> 1, n = c & 1;
      const uint32_t scv = h ? sc47 : sc03;
      const uint32_t sl = splat_byte_u16x2(scv & 0x07070707u, jb0 + n);
      const uint32_t sh = splat_byte_u16x2((scv >> 3) & 0x07070707u, jb0 + n);
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t v = raw[4 + 4 * h + d];
        const uint32_t nib = n ? q4k_hi_nibbles(v) : q4k_lo_nibbles(v);
        lo[d] = pkmul(nib, sl);
        hi[d] = pkmul(nib, sh);
      }
      alo[c] = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
      ahi[c] = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    return f16_bits_to_f32(raw[0]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int h = c >> 1, n = c & 1;
      // scale index 8h + 4n + g4: byte g4 of scale dword 2h + n
      uint32_t s2, c64;
      q6_scale(raw[16 + 2 * h + n], g4, s2, c64);
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t ql = raw[4 * h + d], qh = raw[8 + 4 * h + d];
        const uint32_t q = n ? q6_quants<1>(ql, qh, g4) : q6_quants<0>(ql, qh, g4);
        q6_planes(q, s2, c64, lo[d], hi[d]);
      }
      alo[c] = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
      ahi[c] = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    return f16_bits_to_f32(raw[20]);
  }
}

// The same unpacking one K chunk c (0..3) at a time, so that it can be spread
// between matrix instructions: the two int8 planes of chunk c's 16x64 A
// fragment.  Q4_K takes the block's scale bytes sc03/sc47 (q4k_scales of
// raw[1..3]).
template <int QT>
__device__ __forceinline__ void unpack_chunk(const uint32_t (&raw)[QTr<QT>::RAW], int g4, int c,
                                             uint32_t sc03, uint32_t sc47, v4i& alo, v4i& ahi) {
  const int h = c >> 1, n = c & 1;
  uint32_t lo[4], hi[4];
  if constexpr (QT == QT_Q4K) {
    const int jb0 = 2 * (g4 >> 1);
    const uint32_t scv = h ? sc47 : sc03;
    const uint32_t sl = splat_byte_u16x2(scv & 0x07070707u, jb0 + n);
    const uint32_t sh = splat_byte_u16x2((scv >> 3) & 0x07070707u, jb0 + n);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t v = raw[4 + 4 * h + d];
      const uint32_t nib = n ? q4k_hi_nibbles(v) : q4k_lo_nibbles(v);
      lo[d] = pkmul(nib, sl);
      hi[d] = pkmul(nib, sh);
    }
  } else {
    uint32_t s2, c64;
    q6_scale(raw[16 + 2 * h + n], g4, s2, c64);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t ql = raw[4 * h + d], qh = raw[8 + 4 * h + d];
      const uint32_t q = n ? q6_quants<1>(ql, qh, g4) : q6_quants<0>(ql, qh, g4);
      q6_planes(q, s2, c64, lo[d], hi[d]);
    }
  }
  alo = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
  ahi = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ uint32_t f32_order_bits(float v) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Softmax statistics of a set of logits as (m, s): m its largest logit and
// s = sum exp(l - m) (m = -inf, s = 0 for the empty set).  Two sets merge by
// rescaling both sums to the larger maximum, so the per-row statistics can be
// gathered over waves and work-groups in any grouping; the log-sum-exp is
// m + log s and the softmax probability of the largest logit 1 / s.
__device__ __forceinline__ void softmax_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -__builtin_inff()) return;  // both empty
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}
// four logits of which those with ok[i] belong to the set
__device__ __forceinline__ void softmax_add4(float& m, float& s, const float (&l)[4], const bool (&ok)[4]) {
  float m4 = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) m4 = ok[i] ? fmaxf(m4, l[i]) : m4;
  if (m4 == -__builtin_inff()) return;
  float s4 = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s4 += ok[i] ? expf(l[i] - m4) : 0.0f;
  softmax_merge(m, s, m4, s4);
}
// merge over the four 16-lane groups of a wave (lanes r, r + 16, r + 32, r + 48)
__device__ __forceinline__ void softmax_merge_groups(float& m, float& s) {
  softmax_merge(m, s, __shfl_xor(m, 16), __shfl_xor(s, 16));
  softmax_merge(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32));
}

}  // namespace dllm
