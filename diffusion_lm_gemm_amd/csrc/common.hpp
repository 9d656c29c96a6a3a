// Device-side helpers shared by the libdllm kernels (gfx950 / CDNA4 only).
//
// Bit layouts are the GGUF super-block definitions (the mojo-dllm pages name
// Q4_K, Q6_K and Q8_K but print no layout; Development plan, "Corrections to
// the spec" and "Compute design"):
//   Q4_K (144 B): f16 d | f16 dmin | 12 B of 6-bit scales/mins | 128 B nibbles
//   Q6_K (210 B): 128 B low nibbles | 64 B high 2-bit pairs | 16 int8 scales | f16 d
//   Q8_K (292 B): f32 d | 256 int8 | 16 int16 sums of 16
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

constexpr int QK = 256;
constexpr int Q4K_BYTES = 144;
constexpr int Q6K_BYTES = 210;
constexpr int Q8K_BYTES = 292;
constexpr int DEC_BYTES = 356;
constexpr int QT_Q4K = 12;
constexpr int QT_Q6K = 14;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes); loads outside read as 0.
// Descriptor word 3 (0x00020000) is the raw-buffer format for the gfx9 family.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
// soff is wave-uniform (an SGPR): no per-load address arithmetic
__device__ __forceinline__ uint32_t buf_ld32s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ v2u buf_ld64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ v4u buf_ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// Device-coherent 16-byte load and store (cache policy sc1: coherent across
// the XCDs, whose L2 caches are not coherent with each other; the store
// writes through to memory).  For data that one work-group writes and a work
// group on another XCD reads in the same kernel.
constexpr int kCoherentAux = 16;  // sc1
__device__ __forceinline__ v4u buf_ld128_dev(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherentAux);
}
__device__ __forceinline__ void buf_st128_dev(rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCoherentAux);
}
// Wait until every memory access this wave issued has completed (vmcnt 0;
// expcnt and lgkmcnt left alone).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Eight bytes at a 2-byte aligned offset, from dword-aligned loads of only
// the dwords that hold them.
__device__ __forceinline__ void buf_ld64_a2(rsrc_t r, uint32_t off, uint32_t& x0, uint32_t& x1) {
  const uint32_t s = off & 3u, a = off & ~3u;
  const v2u d01 = buf_ld64(r, a);
  const uint32_t d2 = buf_ld32(r, a + (s ? 8u : 4u));
  x0 = __builtin_amdgcn_alignbyte(d01[1], d01[0], s);
  x1 = __builtin_amdgcn_alignbyte(d2, d01[1], s);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xFFFFu));
}

// Split an f32 into f16 halves with hi + lo == a to ~22 bits.  hi keeps the
// top 11 significant bits of a by truncation (exact in f16 for |a| in the
// normal f16 range), and lo is formed from exactly the bits stored in hi:
// the compiler may lower separate f32->f16 conversions with different
// rounding, so hi's value is pinned before it is reused.  a is taken as the
// rounded f32 value the caller passes: with contraction off here, a product
// formed by the caller is never fused into the subtraction, so every kernel
// instantiation splits the same value the same way.
__device__ __forceinline__ void split_f16(float a, _Float16& hi, _Float16& lo) {
#pragma clang fp contract(off)
  const float ht = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xFFFFE000u);
  unsigned short hb = __builtin_bit_cast(unsigned short, (_Float16)ht);
  asm volatile("" : "+v"(hb));
  hi = __builtin_bit_cast(_Float16, hb);
  lo = (_Float16)(a - (float)hi);
}

// Dword at byte address p where p is 2-byte aligned (Q6_K blocks are 210 B,
// so odd blocks start 2 bytes past a dword boundary).  Only dwords holding a
// requested byte are read, so the read never leaves the block.
__device__ __forceinline__ uint32_t ld_u32_a2(const uint8_t* p) {
  const uintptr_t a = (uintptr_t)p;
  const uint32_t* q = (const uint32_t*)(a & ~(uintptr_t)3);
  const uint32_t s = (uint32_t)(a & 3);  // 0 or 2
  const uint32_t lo = q[0];
  const uint32_t hi = q[s ? 1 : 0];
  return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// Two consecutive dwords at a 2-byte aligned byte address.
__device__ __forceinline__ void ld_u64_a2(const uint8_t* p, uint32_t& x0, uint32_t& x1) {
  const uintptr_t a = (uintptr_t)p;
  const uint32_t* q = (const uint32_t*)(a & ~(uintptr_t)3);
  const uint32_t s = (uint32_t)(a & 3);
  const uint32_t d0 = q[0], d1 = q[1];
  const uint32_t d2 = q[s ? 2 : 1];
  x0 = __builtin_amdgcn_alignbyte(d1, d0, s);
  x1 = __builtin_amdgcn_alignbyte(d2, d1, s);
}

// ---- Q4_K ---------------------------------------------------------------
// Scale/min bytes S[0..11] arrive as three dwords h1 = S[0..3], h2 = S[4..7],
// h3 = S[8..11].  Sub-blocks 0..3: scale = S[j] & 63, min = S[j+4] & 63.
// Sub-blocks 4..7: low 4 bits in the nibbles of S[j+4], top 2 bits in the
// spare bits 6..7 of S[j-4] (scale) and S[j] (min).  Results: one byte per
// sub-block, sc03/mn03 for sub-blocks 0..3 and sc47/mn47 for 4..7.
__device__ __forceinline__ void q4k_scales(uint32_t h1, uint32_t h2, uint32_t h3,
                                           uint32_t& sc03, uint32_t& sc47,
                                           uint32_t& mn03, uint32_t& mn47) {
  sc03 = h1 & 0x3F3F3F3Fu;
  mn03 = h2 & 0x3F3F3F3Fu;
  sc47 = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
  mn47 = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
}

// The 4-bit quants of one dword of the nibble area: low nibbles belong to the
// even sub-block of the 32-byte run, high nibbles to the odd one.
__device__ __forceinline__ uint32_t q4k_lo_nibbles(uint32_t v) { return v & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t q4k_hi_nibbles(uint32_t v) { return (v >> 4) & 0x0F0F0F0Fu; }

// ---- Q6_K ---------------------------------------------------------------
// Four 6-bit quants (one per byte) of quarter k (0..3) from a dword of the
// low-nibble area (taken at 64h + 32(k&1) + l) and the dword of the high-bit
// area at 32h + l: low 4 bits are the low nibble for k < 2 and the high nibble
// for k >= 2; the top 2 bits are bits 2k..2k+1 of the high-bit byte.
__device__ __forceinline__ uint32_t q6k_quants(uint32_t ql, uint32_t qh, int k) {
  const uint32_t lo4 = (ql >> (4 * (k >> 1))) & 0x0F0F0F0Fu;
  const uint32_t hi2 = (qh >> (2 * k)) & 0x03030303u;
  return lo4 | (hi2 << 4);
}

// Byte j (0..3) of x splatted into both 16-bit halves.
__device__ __forceinline__ uint32_t splat_byte_u16x2(uint32_t x, int j) {
  const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)j << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(0u, x, sel);
}

__device__ __forceinline__ u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t as_u32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }

}  // namespace dllm
