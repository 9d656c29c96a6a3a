// Quantized GEMM Q8_K x {Q4_K, Q6_K} on CDNA4 MFMA, with the masked-row LM
// head's argmax epilogue.
//
// What is computed (mojo-dllm Development plan, "Compute design"): every
// linear layer of a denoising step multiplies L per-token Q8_K activation rows
// by GGUF weight rows; with x_hat = d_x q and w_hat the dequantized weights,
//   y[m][n] = sum_sb d_x[m,sb] * sum_{i<256} w_hat[n, 256 sb + i] q[m, 256 sb + i].
// The pages' CPU micro-kernel works on the shared form (unsigned bytes, an
// int16 scale per 16, an f32 offset per 16).  On gfx950 the same sums are
// arranged for the matrix cores:
//
//  * Integer sub-block scales are folded into the weight operand while it is
//    unpacked in registers, as two exact int8 planes:
//      Q4_K: sc*u = 8*(sh*u) + (sl*u), sc = 8 sh + sl, so both planes <= 105;
//      Q6_K: s*(q-32) = 128*hi + lo, lo in [0,127], hi in [-32,32].
//    Two v_mfma_i32_16x16x64_i8 per 64-wide K chunk give the exact int32
//    super-block dot A_sb = (hi << shift) + lo (|A_sb| < 2^31).
//  * The super-block epilogue in f32: y += (d * d_x) * A_sb.
//  * Q4_K's min term -dmin * sum_j m_j * (bsum_{2j} + bsum_{2j+1}) * d_x is a
//    K/32-long contraction; its operands (-dmin*m_j exact in two f16 halves,
//    d_x*S_j split into two f16 halves) go through v_mfma_f32_16x16x32_f16
//    straight into the f32 output accumulator, four super-blocks per MFMA, so
//    it needs no per-super-block epilogue.  Per token, d_x is pre-scaled by a
//    power of two so the f16 halves cannot overflow; the output is scaled back
//    exactly at the end.
//
// Work-group: 256 threads = 4 waves, 64 weight rows (16 per wave) x up to 160
// tokens (TB blocks of 16).  Activations of one super-block are staged in LDS
// and shared by the 4 waves; each wave unpacks only its own 16 rows.  K may be
// split across work-groups (grid.y); partial tiles then go to a workspace and a
// second kernel sums them in split order.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {

constexpr int ACT_STRIDE = 272;  // LDS bytes per token row (256 + 16: spreads banks)

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
  static constexpr int RAW = 17;
};



__device__ __forceinline__ uint32_t pkmul(uint32_t a, uint32_t b) {
  return as_u32(as_u16x2(a) * as_u16x2(b));
}

// Raw (packed) bytes of the lane's part of one weight super-block at byte
// offset `off` of the weight buffer.  Reads past the end of the buffer (rows
// beyond N) return zeros, so padded rows contribute nothing.
template <int QT>
__device__ __forceinline__ void load_raw(rsrc_t wr, uint32_t off, int g4, uint32_t (&raw)[QTr<QT>::RAW]) {
  if constexpr (QT == QT_Q4K) {
    // header (d | dmin, 12 scale/min bytes) and, per chunk c, the 8 nibble
    // bytes at 16 + 32c + 8 g4.
    const v4u hdr = buf_ld128(wr, off);
    raw[0] = hdr[0]; raw[1] = hdr[1]; raw[2] = hdr[2]; raw[3] = hdr[3];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v2u v = buf_ld64(wr, off + 16 + 32 * c + 8 * g4);
      raw[4 + 2 * c] = v[0];
      raw[5 + 2 * c] = v[1];
    }
  } else {
    // per chunk c = (half h, quarter pair k1): low-nibble bytes at
    // 64h + 32k1 + 8 g4; per half: high-bit bytes at 128 + 32h + 8 g4;
    // 16 scale bytes at 192; f16 d at 208.  Blocks are 210 bytes, so a block
    // may start 2 bytes past a dword boundary.
#pragma unroll
    for (int c = 0; c < 4; ++c) buf_ld64_a2(wr, off + 64 * (c >> 1) + 32 * (c & 1) + 8 * g4, raw[2 * c], raw[2 * c + 1]);
#pragma unroll
    for (int h = 0; h < 2; ++h) buf_ld64_a2(wr, off + 128 + 32 * h + 8 * g4, raw[8 + 2 * h], raw[9 + 2 * h]);
    buf_ld64_a2(wr, off + 192, raw[12], raw[13]);
    buf_ld64_a2(wr, off + 200, raw[14], raw[15]);
    raw[16] = buf_ld16(wr, off + 208);
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

// Unpack raw bytes into the two int8 planes of the four 16x64 A fragments and
// return the super-block factor d.
template <int QT>
__device__ __forceinline__ float unpack(const uint32_t (&raw)[QTr<QT>::RAW], int g4, v4i (&alo)[4], v4i (&ahi)[4]) {
  if constexpr (QT == QT_Q4K) {
    uint32_t sc03, sc47, mn03, mn47;
    q4k_scales(raw[1], raw[2], raw[3], sc03, sc47, mn03, mn47);
    const uint32_t sl03 = sc03 & 0x07070707u, sh03 = (sc03 >> 3) & 0x07070707u;
    const uint32_t sl47 = sc47 & 0x07070707u, sh47 = (sc47 >> 3) & 0x07070707u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // sub-blocks 2c (low nibbles) and 2c+1 (high nibbles)
      const uint32_t slv = (c < 2) ? sl03 : sl47, shv = (c < 2) ? sh03 : sh47;
      const int je = (2 * c) & 3, jo = (2 * c + 1) & 3;
      const uint32_t sle = splat_byte_u16x2(slv, je), slo = splat_byte_u16x2(slv, jo);
      const uint32_t she = splat_byte_u16x2(shv, je), sho = splat_byte_u16x2(shv, jo);
      const uint32_t v0 = raw[4 + 2 * c], v1 = raw[5 + 2 * c];
      const uint32_t n0l = q4k_lo_nibbles(v0), n1l = q4k_lo_nibbles(v1);
      const uint32_t n0h = q4k_hi_nibbles(v0), n1h = q4k_hi_nibbles(v1);
      alo[c] = v4i{(int)pkmul(n0l, sle), (int)pkmul(n1l, sle), (int)pkmul(n0h, slo), (int)pkmul(n1h, slo)};
      ahi[c] = v4i{(int)pkmul(n0l, she), (int)pkmul(n1l, she), (int)pkmul(n0h, sho), (int)pkmul(n1h, sho)};
    }
    return f16_bits_to_f32(raw[0]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int h = c >> 1, k1 = c & 1;
      // scale index g = i/16 for quarters k1 and k1+2 at l = 8 g4 .. 8 g4 + 7
      const int gl = 8 * h + 2 * k1 + (g4 >> 1), gh = gl + 4;
      const int sl = (int)(int8_t)(raw[12 + (gl >> 2)] >> (8 * (gl & 3)));
      const int sh = (int)(int8_t)(raw[12 + (gh >> 2)] >> (8 * (gh & 3)));
      const uint32_t s2l = ((uint32_t)(2 * sl) & 0xFFFFu) * 0x10001u;
      const uint32_t c64l = ((uint32_t)(-64 * sl) & 0xFFFFu) * 0x10001u;
      const uint32_t s2h = ((uint32_t)(2 * sh) & 0xFFFFu) * 0x10001u;
      const uint32_t c64h = ((uint32_t)(-64 * sh) & 0xFFFFu) * 0x10001u;
      const uint32_t L0 = raw[2 * c], L1 = raw[2 * c + 1];
      const uint32_t H0 = raw[8 + 2 * h], H1 = raw[9 + 2 * h];
      uint32_t lo[4], hi[4];
      q6_planes(q6k_quants(L0, H0, k1), s2l, c64l, lo[0], hi[0]);
      q6_planes(q6k_quants(L1, H1, k1), s2l, c64l, lo[1], hi[1]);
      q6_planes(q6k_quants(L0, H0, k1 + 2), s2h, c64h, lo[2], hi[2]);
      q6_planes(q6k_quants(L1, H1, k1 + 2), s2h, c64h, lo[3], hi[3]);
      alo[c] = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
      ahi[c] = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    return f16_bits_to_f32(raw[16]);
  }
}

// LDS layout of one token's 256 activation bytes: the 16 bytes that pair
// with lane group g4 of K chunk c (in the A fragment's K order) sit together
// at byte 16 (4c + g4), so each B fragment is one 16-byte LDS read.  With a
// 272-byte token stride the 16-byte reads of a wave fall in distinct banks.
// act_dst maps the natural byte offset o (a multiple of 4) to that layout.
template <int QT>
__device__ __forceinline__ int act_dst(int o) {
  int c, piece, l;
  if constexpr (QT == QT_Q4K) {  // chunk c = bytes 64c..64c+63: two 32-byte pieces
    c = o >> 6;
    piece = (o >> 5) & 1;
    l = o & 31;
  } else {  // chunk c = (half h, quarter k & 1); piece = k >> 1
    const int h = o >> 7, k = (o >> 5) & 3;
    c = 2 * h + (k & 1);
    piece = k >> 1;
    l = o & 31;
  }
  return (4 * c + (l >> 3)) * 16 + piece * 8 + (l & 7);
}

__device__ __forceinline__ uint32_t f32_order_bits(float v) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// NW waves per work-group, RB row blocks of 16 weight rows per wave: the tile
// is 16 * RB * NW rows x 16 * TB tokens.  Each B fragment read from LDS feeds
// 2 * RB MFMAs, so RB = 2 halves the LDS traffic per MFMA.
template <int QT, int TB, int NW, int RB, bool ARGMAX>
__global__ __launch_bounds__(64 * NW, 1) void k_qgemm(GemmParams p) {
  constexpr int TOK = TB * 16;          // tokens per work-group (MFMA columns)
  constexpr int NTH = 64 * NW;          // threads
  constexpr int ROWS = 16 * RB * NW;    // weight rows per work-group
  constexpr int STG = TOK / NW;         // activation dwords per thread per stage
  constexpr int SHIFT = QTr<QT>::SHIFT;
  constexpr int BYTES = QTr<QT>::BYTES;
  constexpr int RAW = QTr<QT>::RAW;
  constexpr bool MINS = (QT == QT_Q4K);
  // Two activation stages (double buffer), their d_x, and for Q4_K an 8-slot
  // ring (two groups of four super-blocks) of min-term activation operands
  // [slot][token][hi8 | lo8] f16: one group is read while the next is written.
  __shared__ __attribute__((aligned(16))) uint8_t s_act[2][TOK * ACT_STRIDE];
  // d_x staging: item i (a token, or a (token, j) pair for Q4_K) writes
  // slot i, so every store has its own address; token t's value is read at
  // item t * DXS.  Items past the end write the tail, which nothing reads.
  constexpr int NITEM = MINS ? TOK * 8 : TOK;
  constexpr int IPT = (NITEM + NTH - 1) / NTH;  // items per thread
  constexpr int DXS = MINS ? 8 : 1;
  __shared__ float s_dx[2][IPT * NTH];
  __shared__ float s_esc[TOK];
  __shared__ __attribute__((aligned(16))) _Float16 s_amin[MINS ? 8 * TOK * 16 + 2 * (IPT * NTH - NITEM) + 8 : 8];
  __shared__ uint64_t s_key[ARGMAX ? NW * TOK : 1];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t N = p.N, SB = p.SB, M = p.M;
  const int64_t m0 = (int64_t)blockIdx.z * TOK;
  const int64_t s0 = (int64_t)blockIdx.y * p.sps;
  const int64_t s1 = (s0 + p.sps < SB) ? s0 + p.sps : SB;
  const int64_t row0 = (int64_t)blockIdx.x * ROWS + wv * 16 * RB;  // first row of this wave
  // Buffer resources: loads past num_records read as zero (rows >= N,
  // tokens >= M).  The host keeps both operands below 2 GiB.
  const rsrc_t wr = make_rsrc(p.w, N * SB * BYTES);
  const rsrc_t xr = make_rsrc(p.xq, M * SB * Q8K_BYTES);
  uint32_t wrow_off[RB];
  bool row_ok[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int64_t nrow = row0 + 16 * b + r;  // the row this lane unpacks
    row_ok[b] = nrow < N;
    wrow_off[b] = (uint32_t)(nrow * SB * BYTES);
  }

  // Per-token power-of-two pre-scale of d_x (Q4_K: keeps the f16 halves of
  // d_x * S_j in range; undone exactly at the end); 1 for Q6_K.
  if (tid < TOK) {
    float esc = 1.0f;
    if constexpr (MINS) {
      // eight independent loads in flight per round
      float mx = 0.0f;
      const uint32_t tok_off = (uint32_t)((m0 + tid) * SB * Q8K_BYTES);
      for (int64_t sb = s0; sb < s1; sb += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_bit_cast(float, buf_ld32(xr, tok_off + (uint32_t)((sb + u) * Q8K_BYTES)));
#pragma unroll
        for (int u = 0; u < 8; ++u) mx = (sb + u < s1) ? fmaxf(mx, __builtin_fabsf(v[u])) : mx;
      }
      if (mx > 0.0f) {
        int e = 0;
        (void)frexpf(mx, &e);
        e = e < -100 ? -100 : (e > 100 ? 100 : e);
        esc = ldexpf(1.0f, -e);
      }
    }
    s_esc[tid] = esc;
  }
  if constexpr (MINS) {
    for (int i = tid; i < 8 * TOK * 16; i += NTH) s_amin[i] = (_Float16)0.0f;
  }
  __syncthreads();

  // ---- activation staging: global -> registers (issued one super-block
  // ahead) -> LDS.  Thread tid moves dword (tid & 63) of tokens wv + NW k,
  // placing it by act_dst.  d_x (and for Q4_K the min-term operands, one
  // (token, j) pair per item) are spread over all threads.  Every load is
  // unconditional -- past the end of the operand the buffer reads zero -- and
  // so is every store (to its own LDS address): a fixed load count keeps the
  // wait counts exact, and no branch lets the compiler sink the loads next to
  // their use at the end of the iteration.
  const uint32_t act_step = (uint32_t)(NW * SB * Q8K_BYTES);
  const int dcol = tid & 63;
  const int dst_col = act_dst<QT>(4 * dcol);
  uint32_t av[STG];
  uint32_t idx_d[IPT], idx_b[IPT];
  auto act_load = [&](int64_t sb) {
    const uint32_t base = (uint32_t)(((m0 + wv) * SB + sb) * Q8K_BYTES) + 4 + 4 * dcol;
#pragma unroll
    for (int k = 0; k < STG; ++k) av[k] = buf_ld32s(xr, base, k * act_step);
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int item = tid + k * NTH;
      const int it_c = item < NITEM ? item : NITEM - 1;
      const int tok = MINS ? (it_c >> 3) : it_c;
      const uint32_t xoff = (uint32_t)(((m0 + tok) * SB + sb) * Q8K_BYTES);
      idx_d[k] = buf_ld32(xr, xoff);
      if constexpr (MINS) idx_b[k] = buf_ld32(xr, xoff + 260 + 4 * (it_c & 7));
    }
  };
  auto act_store = [&](int buf, int slot8) {
    uint8_t* dst = s_act[buf] + wv * ACT_STRIDE + dst_col;
#pragma unroll
    for (int k = 0; k < STG; ++k) *(uint32_t*)(dst + k * NW * ACT_STRIDE) = av[k];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int item = tid + k * NTH;
      const bool live = item < NITEM;
      const int it_c = live ? item : NITEM - 1;
      const int tok = MINS ? (it_c >> 3) : it_c;
      const float dx = __builtin_bit_cast(float, idx_d[k]) * s_esc[tok];
      s_dx[buf][item] = dx;
      if constexpr (MINS) {
        // activation side of the min term: d_x * (bsum_{2j} + bsum_{2j+1}),
        // as f16 high and low halves
        const int j = it_c & 7;
        const uint32_t pr = idx_b[k];
        const int S = (int)(int16_t)(pr & 0xFFFFu) + (int)(int16_t)(pr >> 16);
        _Float16* dm_hi = s_amin + (live ? (slot8 * TOK + tok) * 16 + j : 8 * TOK * 16 + 2 * (item - NITEM));
        _Float16* dm_lo = live ? dm_hi + 8 : dm_hi + 1;
        split_f16(dx * (float)S, *dm_hi, *dm_lo);
      }
    }
  };

  v4f yacc[RB][TB];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int t = 0; t < TB; ++t) yacc[b][t] = v4f{0.f, 0.f, 0.f, 0.f};
  // Q4_K: dmin and min bytes of block (group start + g4) of each row, taken
  // from the lane's own block data when the loop passes that super-block
  uint32_t mh0[RB], mh2[RB], mh3[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) mh0[b] = mh2[b] = mh3[b] = 0u;

  // One super-block: stage the next activations, unpack this block's weights
  // (loaded two super-blocks ago into `raw`, which is then refilled with the
  // block two ahead), contract on MFMA, fold in the min term at the end of a
  // group of four, publish the next stage.
  auto step = [&](int64_t sb, uint32_t(&raw)[RB][RAW]) {
    const int it = (int)(sb - s0);
    const int buf = it & 1, slot = it & 3;
    const bool more = sb + 1 < s1;
    act_load(sb + 1);
    v4i alo[RB][4], ahi[RB][4];
    float dsel[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const float drow = unpack<QT>(raw[b], g4, alo[b], ahi[b]);
      if constexpr (MINS) {
        const bool mine = (slot == g4);
        mh0[b] = mine ? raw[b][0] : mh0[b];
        mh2[b] = mine ? raw[b][2] : mh2[b];
        mh3[b] = mine ? raw[b][3] : mh3[b];
      }
      load_raw<QT>(wr, wrow_off[b] + (uint32_t)((sb + 2) * BYTES), g4, raw[b]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dsel[b][i] = __shfl(drow, 4 * g4 + i);
    }

    // integer contraction (two planes x four K chunks x RB row blocks) and
    // the super-block epilogue y += (d * d_x) * ((hi << shift) + lo),
    // software-pipelined over the token blocks: the B fragments of block t+1
    // are read while block t's MFMAs run, and block t-1's integer sums are
    // folded into y meanwhile.
    const uint8_t* act = s_act[buf];
    auto loadB = [&](int t, v4i(&dstB)[4]) {
      const uint8_t* arow = act + (t * 16 + r) * ACT_STRIDE + g4 * 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) dstB[c] = *(const v4i*)(arow + 64 * c);
    };
    auto flush = [&](int t, const v4i(&al)[RB], const v4i(&ah)[RB]) {
      const float dx = s_dx[buf][(t * 16 + r) * DXS];
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = (ah[b][i] << SHIFT) + al[b][i];
          yacc[b][t][i] += (float)a * (dsel[b][i] * dx);
        }
    };
    v4i Bc[4], Bn[4];
    loadB(0, Bc);
    v4i pl[RB], ph[RB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t + 1 < TB) loadB(t + 1, Bn);
      v4i al[RB], ah[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) al[b] = ah[b] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          al[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[b][c], Bc[c], al[b], 0, 0, 0);
          ah[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi[b][c], Bc[c], ah[b], 0, 0, 0);
        }
      if (t > 0) flush(t - 1, pl, ph);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        pl[b] = al[b];
        ph[b] = ah[b];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) Bc[c] = Bn[c];
    }
    flush(TB - 1, pl, ph);

    // Q4_K min term, once per group of four super-blocks (or at the end);
    // lanes whose super-block lies past the end contribute zero
    if constexpr (MINS) {
      if (slot == 3 || !more) {
        v8h bmin_hi[RB], bmin_lo[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const bool live = row_ok[b] && g4 <= slot;
          uint32_t sc03, sc47, mn03, mn47;
          q4k_scales(0u, live ? mh2[b] : 0u, live ? mh3[b] : 0u, sc03, sc47, mn03, mn47);
          const float ndmin = -f16_bits_to_f32(live ? (mh0[b] >> 16) : 0u);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t mb = (j < 4) ? mn03 : mn47;
            _Float16 hi, lo;
            split_f16(ndmin * (float)((mb >> (8 * (j & 3))) & 63u), hi, lo);
            bmin_hi[b][j] = hi;
            bmin_lo[b][j] = lo;
          }
        }
        const int gbase = (it & 4);  // ring slots of this group: gbase .. gbase + 3
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const _Float16* src = s_amin + ((gbase + g4) * TOK + t * 16 + r) * 16;
          const v8h ahv = *(const v8h*)src;
          const v8h alv = *(const v8h*)(src + 8);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            yacc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_hi[b], ahv, yacc[b][t], 0, 0, 0);
            yacc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_hi[b], alv, yacc[b][t], 0, 0, 0);
            yacc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_lo[b], ahv, yacc[b][t], 0, 0, 0);
          }
        }
      }
    }
    act_store(buf ^ 1, (it + 1) & 7);  // past the end: an unread stage
    __syncthreads();
  };

  // ---- prologue: weights for the first two super-blocks, first stage
  uint32_t rawA[RB][RAW], rawB[RB][RAW];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    load_raw<QT>(wr, wrow_off[b] + (uint32_t)(s0 * BYTES), g4, rawA[b]);
    load_raw<QT>(wr, wrow_off[b] + (uint32_t)((s0 + 1) * BYTES), g4, rawB[b]);
  }
  act_load(s0);
  act_store(0, 0);
  __syncthreads();

  int64_t sb = s0;
  for (; sb + 1 < s1; sb += 2) {
    step(sb, rawA);
    step(sb + 1, rawB);
  }
  if (sb < s1) step(sb, rawA);

  // ---- write out: lane holds rows nbase + i (i < 4) of token t*16 + r
  float* outp = p.out + (int64_t)blockIdx.y * p.split_stride;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int64_t nbase = row0 + 16 * b + 4 * g4;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int64_t m = m0 + t * 16 + r;
      const float inv = 1.0f / s_esc[t * 16 + r];  // exact: a power of two
      const v4f yv = yacc[b][t] * inv;
      yacc[b][t] = yv;
      if (m < M) {
        float* dst = outp + m * p.ldo + nbase;
        if (nbase + 3 < N && ((((uintptr_t)dst) & 15) == 0)) {
          *(v4f*)dst = yv;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nbase + i < N) dst[i] = yv[i];
        }
      }
    }
  }

  if constexpr (ARGMAX) {
    // per token: best (value, lowest row index) over this work-group's rows
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      uint64_t best = 0;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t n = row0 + 16 * b + 4 * g4 + i;
          if (n < N) {
            const uint64_t key = ((uint64_t)f32_order_bits(yacc[b][t][i]) << 32) | (uint64_t)(~(uint32_t)n);
            best = key > best ? key : best;
          }
        }
      const uint64_t o1 = __shfl_xor(best, 16);
      best = o1 > best ? o1 : best;
      const uint64_t o2 = __shfl_xor(best, 32);
      best = o2 > best ? o2 : best;
      if (g4 == 0) s_key[wv * TOK + t * 16 + r] = best;
    }
    __syncthreads();
    if (tid < TOK) {
      const int64_t m = m0 + tid;
      uint64_t best = s_key[tid];
#pragma unroll
      for (int k = 1; k < NW; ++k) best = s_key[k * TOK + tid] > best ? s_key[k * TOK + tid] : best;
      if (m < M) p.keys[(int64_t)blockIdx.x * M + m] = best;
    }
  }
}

// Sum of the K-split partial tiles in split order (deterministic).
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ ws, int S, int64_t M,
                                                    int64_t N, float* __restrict__ y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i - m * N;
  float acc = ws[i];
  for (int s = 1; s < S; ++s) acc += ws[(int64_t)s * M * N + i];
  y[m * ldy + n] = acc;
}

// argmax[m] = lowest row index of the largest logit, from per-tile keys.
__global__ __launch_bounds__(256) void k_argmax_finalize(const uint64_t* __restrict__ keys, int64_t n_tiles,
                                                       int64_t M, int32_t* __restrict__ argmax) {
  __shared__ uint64_t red[256];
  const int64_t m = blockIdx.x;
  uint64_t best = 0;
  for (int64_t t = threadIdx.x; t < n_tiles; t += 256) {
    const uint64_t k = keys[t * M + m];
    best = k > best ? k : best;
  }
  red[threadIdx.x] = best;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s && red[threadIdx.x + s] > red[threadIdx.x]) red[threadIdx.x] = red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) argmax[m] = (int32_t)(~(uint32_t)(red[0] & 0xFFFFFFFFu));
}

// Test export: per-16 integer partial dots of the unsigned shared-form quants
// with the Q8_K quants, through the same bit unpacking as the GEMM.
template <int QT>
__global__ __launch_bounds__(256) void k_partials(const uint8_t* __restrict__ w, int64_t N, int64_t SB,
                                                const uint8_t* __restrict__ xq, int64_t M,
                                                int32_t* __restrict__ P) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N * SB * 16) return;
  const int g = (int)(i & 15);
  const int64_t sb = (i >> 4) % SB;
  const int64_t n = ((i >> 4) / SB) % N;
  const int64_t m = (i >> 4) / (SB * N);
  const uint8_t* xr = xq + (m * SB + sb) * Q8K_BYTES + 4 + 16 * g;
  int acc = 0;
  for (int d = 0; d < 4; ++d) {
    uint32_t u;
    if constexpr (QT == QT_Q4K) {
      const uint8_t* b = w + (n * SB + sb) * Q4K_BYTES;
      const int j = g >> 1;
      const uint32_t v = *(const uint32_t*)(b + 16 + 32 * (j >> 1) + 16 * (g & 1) + 4 * d);
      u = (j & 1) ? q4k_hi_nibbles(v) : q4k_lo_nibbles(v);
    } else {
      const uint8_t* b = w + (n * SB + sb) * Q6K_BYTES;
      const int h = g >> 3, k = (g >> 1) & 3, l = 16 * (g & 1) + 4 * d;
      u = q6k_quants(ld_u32_a2(b + 64 * h + 32 * (k & 1) + l), ld_u32_a2(b + 128 + 32 * h + l), k);
    }
    const uint32_t q = *(const uint32_t*)(xr + 4 * d);
    acc = __builtin_amdgcn_sdot4((int)q, (int)u, acc, false);  // u <= 63 is also a valid int8
  }
  P[i] = acc;
}

// ---- host-side launch helpers -------------------------------------------
template <int QT, int TB, int NW, int RB, bool ARGMAX>
static hipError_t launch_k(const GemmParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_qgemm<QT, TB, NW, RB, ARGMAX>), grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

template <int QT, int NW, int RB, bool ARGMAX>
static hipError_t launch_q(const GemmParams& p, int tb, dim3 grid, hipStream_t s) {
  switch (tb) {
    case 1: return launch_k<QT, 1, NW, RB, ARGMAX>(p, grid, s);
    case 2: return launch_k<QT, 2, NW, RB, ARGMAX>(p, grid, s);
    case 3: return launch_k<QT, 3, NW, RB, ARGMAX>(p, grid, s);
    case 4: return launch_k<QT, 4, NW, RB, ARGMAX>(p, grid, s);
    case 5: return launch_k<QT, 5, NW, RB, ARGMAX>(p, grid, s);
    case 6: return launch_k<QT, 6, NW, RB, ARGMAX>(p, grid, s);
    case 7: return launch_k<QT, 7, NW, RB, ARGMAX>(p, grid, s);
    case 8: return launch_k<QT, 8, NW, RB, ARGMAX>(p, grid, s);
    case 9: return launch_k<QT, 9, NW, RB, ARGMAX>(p, grid, s);
    default: return launch_k<QT, 10, NW, RB, ARGMAX>(p, grid, s);
  }
}

// Tile configurations: cfg 0 = 4 waves x 2 row blocks (128 rows, one wave per
// SIMD), cfg 1 = 4 waves x 1 row block (64 rows), cfg 2 = 8 waves x 1 row
// block (128 rows, two waves per SIMD).  The LM head (argmax) uses cfg 1.
template <int QT>
static hipError_t launch_cfg(const GemmParams& p, int tb, int cfg, dim3 grid, bool argmax, hipStream_t s) {
  if (argmax) return launch_q<QT, 4, 1, true>(p, tb, grid, s);
  if (cfg == 0) return launch_q<QT, 4, 2, false>(p, tb, grid, s);
  if (cfg == 1) return launch_q<QT, 4, 1, false>(p, tb, grid, s);
  return launch_q<QT, 8, 1, false>(p, tb, grid, s);
}

int qgemm_cfg_rows(int cfg) { return cfg == 1 ? 64 : 128; }

hipError_t launch_qgemm(int qtype, const GemmParams& p, int tb, int cfg, dim3 grid, bool argmax, hipStream_t s) {
  if (qtype == QT_Q4K) return launch_cfg<QT_Q4K>(p, tb, cfg, grid, argmax, s);
  return launch_cfg<QT_Q6K>(p, tb, cfg, grid, argmax, s);
}

hipError_t launch_split_reduce(const float* ws, int S, int64_t M, int64_t N, float* y, int64_t ldy, hipStream_t s) {
  const int64_t total = M * N;
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, ws, S, M, N, y, ldy);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(const uint64_t* keys, int64_t n_tiles, int64_t M, int32_t* argmax, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_finalize, dim3((unsigned)M), dim3(256), 0, s, keys, n_tiles, M, argmax);
  return hipGetLastError();
}

hipError_t launch_partials(int qtype, const uint8_t* w, int64_t N, int64_t SB, const uint8_t* xq, int64_t M,
                           int32_t* P, hipStream_t s) {
  const int64_t total = M * N * SB * 16;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL(k_partials<QT_Q4K>, grid, dim3(256), 0, s, w, N, SB, xq, M, P);
  else
    hipLaunchKernelGGL(k_partials<QT_Q6K>, grid, dim3(256), 0, s, w, N, SB, xq, M, P);
  return hipGetLastError();
}

}  // namespace dllm
