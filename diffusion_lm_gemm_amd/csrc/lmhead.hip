// Masked-row LM head, streaming form: logits and greedy argmax for at most 32
// gathered rows of the hidden state against the whole output matrix.
//
// The LM head runs only on the masked positions of the current block (mojo-
// dllm Development plan, "Compute design", last bullet; README "How it
// works"): at most 32 token rows against 126464 weight rows.  With so few
// tokens the work per weight super-block is small, so a tiled GEMM that
// synchronises its work-group once per super-block spends its time waiting
// for weights.  Here every work-group loads the gathered Q8_K rows into LDS
// once (all of K), and then each wave streams its own 16-row blocks with the
// weights requested three super-blocks ahead and no barrier: one wave's memory
// latency is covered by the others.  The arithmetic is the GEMM's (two int8
// planes on v_mfma_i32_16x16x64_i8, the per-super-block f32 epilogue, and for
// Q4_K the min term on f16 MFMA), and each wave keeps, per token, the largest
// (logit, lowest row) key over its rows.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "unpack.hpp"

namespace dllm {

constexpr int LM_TOK = 32;  // token columns (two MFMA blocks of 16)
constexpr int LM_SBMAX = 16;  // K <= 4096

// Keys are (order-preserving f32 bits << 32) | ~row: the largest key is the
// largest logit, and among equal logits the lowest row.
//
// PARITY (Q6_K with an even number of super-blocks per row): a 210-byte
// block then starts 4-byte aligned exactly when its super-block index is
// even, the same for every lane of a step, and step st of a wave's stream has
// the parity of st.  Even blocks are loaded without the alignment dwords and
// used without byte shifts; the loop runs six steps per iteration so that
// each step's parity and buffer are fixed at compile time.  The stream is
// bound by its vector-memory instructions, of which this removes a quarter.
template <int QT, int NW, bool PARITY>
__global__ __launch_bounds__(64 * NW, 1) void k_lmhead_stream(LmParams p) {
  constexpr int SHIFT = QTr<QT>::SHIFT;
  constexpr int BYTES = QTr<QT>::BYTES;
  constexpr int RAW = QTr<QT>::RAW;
  constexpr int RAWW = QTw<QT>::RAW;  // dword-aligned loads (see load_raw_dw)
  constexpr bool MINS = (QT == QT_Q4K);
  constexpr int NTH = 64 * NW;
  // activations, natural K order per token, 16-byte units XOR-swizzled by
  // token (unit u of token tok at u ^ (tok & 15)); d_x per (token, sb); for
  // Q4_K the min-term operands per (sb, token), high and low f16 halves, for
  // sb up to a multiple of four (the padding is zero).
  __shared__ __attribute__((aligned(16))) uint8_t s_act[LM_TOK * LM_SBMAX * 256];
  __shared__ float s_dx[LM_TOK * LM_SBMAX];
  __shared__ float s_esc[LM_TOK];
  __shared__ __attribute__((aligned(16))) _Float16 s_amh[MINS ? LM_SBMAX * LM_TOK * 8 : 8];
  __shared__ __attribute__((aligned(16))) _Float16 s_aml[MINS ? LM_SBMAX * LM_TOK * 8 : 8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t N = p.N, M = p.M;
  const int SB = (int)p.SB;
  const int KU = SB * 16;  // 16-byte units per token row
  const rsrc_t wr = make_rsrc(p.w, N * SB * BYTES);
  const rsrc_t xr = make_rsrc(p.xq, M * SB * Q8K_BYTES);

  // ---- load the gathered rows (tokens >= M read as zero)
  const int n_units = LM_TOK * KU;
  for (int u0 = wv * 64; u0 < n_units; u0 += NTH) {
    const int U = u0 + lane;
    const int tok = U / KU, slot = U - tok * KU;
    const int gu = slot ^ (tok & 15);
    const uint32_t voff = (uint32_t)((tok * SB + (gu >> 4)) * Q8K_BYTES) + 4 + 16 * (gu & 15);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(s_act + u0 * 16), 16,
                                             voff, 0, 0, 0);
  }
  for (int i = tid; i < LM_TOK * SB; i += NTH) {
    const int tok = i / SB, sb = i - tok * SB;
    s_dx[i] = __builtin_bit_cast(float, buf_ld32(xr, (uint32_t)((tok * SB + sb) * Q8K_BYTES)));
  }
  __syncthreads();
  if constexpr (MINS) {
    // per-token power-of-two pre-scale keeping the f16 halves of d_x * S_j in
    // range (undone exactly in the epilogue)
    if (tid < LM_TOK) {
      float mx = 0.0f;
      for (int sb = 0; sb < SB; ++sb) mx = fmaxf(mx, __builtin_fabsf(s_dx[tid * SB + sb]));
      float esc = 1.0f;
      if (mx > 0.0f) {
        int e = 0;
        (void)frexpf(mx, &e);
        e = e < -100 ? -100 : (e > 100 ? 100 : e);
        esc = ldexpf(1.0f, -e);
      }
      s_esc[tid] = esc;
    }
    __syncthreads();
    const int sbp = (SB + 3) & ~3;
    for (int i = tid; i < sbp * LM_TOK * 8; i += NTH) {
      const int j = i & 7, tok = (i >> 3) % LM_TOK, sb = (i >> 3) / LM_TOK;
      float v = 0.0f;
      if (sb < SB) {
        const uint32_t pr = buf_ld32(xr, (uint32_t)((tok * SB + sb) * Q8K_BYTES) + 260 + 4 * j);
        const int S = (int)(int16_t)(pr & 0xFFFFu) + (int)(int16_t)(pr >> 16);
        v = s_dx[tok * SB + sb] * s_esc[tok] * (float)S;
      }
      split_f16(v, s_amh[i], s_aml[i]);
    }
  } else {
    if (tid < LM_TOK) s_esc[tid] = 1.0f;
  }
  __syncthreads();

  // ---- stream this wave's row blocks: rb = wave, wave + n_waves, ...
  const int64_t n_rb = (N + 15) / 16;
  const int64_t wave = (int64_t)blockIdx.x * NW + wv, n_waves = (int64_t)gridDim.x * NW;
  const int64_t my_rb = wave < n_rb ? (n_rb - wave + n_waves - 1) / n_waves : 0;
  const int64_t n_steps = my_rb * SB;
  // byte offset of super-block sb of this lane's row in row block k
  auto woff = [&](int64_t k, int sb) {
    return (uint32_t)((((wave + k * n_waves) * 16 + r) * SB + sb) * BYTES);
  };
  int bunit[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bunit[c] = act_unit<QT>(c, g4);
  const float esc_t[2] = {s_esc[r], s_esc[16 + r]};

  v4f yacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  uint64_t best[2] = {0, 0};
  // softmax statistics (m, s) per token over the lane's rows (when asked for)
  const bool want_stats = p.stats != nullptr;
  float sm[2] = {-__builtin_inff(), -__builtin_inff()}, ss[2] = {0.0f, 0.0f};
  uint32_t mh0 = 0, mh2 = 0, mh3 = 0;
  int64_t k = 0;   // row block index of this wave's stream
  int sb = 0;      // super-block within it
  int64_t k2 = 0;  // the block three steps ahead
  int sb2 = 0;
  auto advance = [&](int64_t& kk, int& s) {
    if (++s == SB) { s = 0; ++kk; }
  };

  // PAR: 0 = alignment from the offset (any SB), 1 = this block 4-byte
  // aligned and the one three steps ahead not (SB even, sb even), 2 = the
  // other way round
  auto step = [&](auto par_tag, uint32_t(&rw)[RAWW]) {
    constexpr int PAR = decltype(par_tag)::value;
    uint32_t raw[RAW];
    if constexpr (PAR == 1 && QT == QT_Q6K) {
#pragma unroll
      for (int f = 0; f < 5; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[4 * f + i] = rw[5 * f + i];
      raw[20] = rw[25];
    } else {
      align_raw<QT>(rw, woff(k, sb), raw);
    }
    v4i alo[4], ahi[4];
    const float drow = unpack<QT>(raw, g4, alo, ahi);
    if constexpr (MINS) {
      const bool mine = ((sb & 3) == g4);
      mh0 = mine ? raw[0] : mh0;
      mh2 = mine ? raw[2] : mh2;
      mh3 = mine ? raw[3] : mh3;
    }
    // the block three steps ahead (past the end: reads nothing that is used)
    if constexpr (PAR == 2 && QT == QT_Q6K) {
      // 4-byte aligned: the five 16-byte fields and d, no alignment dwords
      const uint32_t off = woff(k2, sb2);
      const uint32_t fo[5] = {off + 16 * g4, off + 64 + 16 * g4, off + 128 + 16 * (g4 & 1), off + 160 + 16 * (g4 & 1),
                              off + 192};
#pragma unroll
      for (int f = 0; f < 5; ++f) {
        const v4u v = buf_ld128(wr, fo[f]);
#pragma unroll
        for (int i = 0; i < 4; ++i) rw[5 * f + i] = v[i];
      }
      rw[25] = buf_ld16(wr, off + 208);
    } else {
      load_raw_dw<QT>(wr, woff(k2, sb2), g4, rw);
    }
    advance(k2, sb2);
    float dsel[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dsel[i] = __shfl(drow, 4 * g4 + i);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* arow = s_act + (t * 16 + r) * (KU * 16) + sb * 256;
      v4i B[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) B[c] = *(const v4i*)(arow + 16 * (bunit[c] ^ r));
      v4i al = {0, 0, 0, 0}, ah = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        al = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[c], B[c], al, 0, 0, 0);
        ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi[c], B[c], ah, 0, 0, 0);
      }
      const float dx = s_dx[(t * 16 + r) * SB + sb] * esc_t[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = (ah[i] << SHIFT) + al[i];
        yacc[t][i] = __builtin_fmaf((float)a, dsel[i] * dx, yacc[t][i]);
      }
    }
    if constexpr (MINS) {
      if ((sb & 3) == 3 || sb == SB - 1) {
        const bool live = g4 <= (sb & 3);
        uint32_t sc03, sc47, mn03, mn47;
        q4k_scales(0u, live ? mh2 : 0u, live ? mh3 : 0u, sc03, sc47, mn03, mn47);
        const float ndmin = -f16_bits_to_f32(live ? (mh0 >> 16) : 0u);
        v8h bh, bl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t mb = (j < 4) ? mn03 : mn47;
          _Float16 hi, lo;
          split_f16(ndmin * (float)((mb >> (8 * (j & 3))) & 63u), hi, lo);
          bh[j] = hi;
          bl[j] = lo;
        }
        const int gbase = sb & ~3;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int o = ((gbase + g4) * LM_TOK + t * 16 + r) * 8;
          const v8h ahv = *(const v8h*)(s_amh + o);
          const v8h alv = *(const v8h*)(s_aml + o);
          yacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, ahv, yacc[t], 0, 0, 0);
          yacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, alv, yacc[t], 0, 0, 0);
          yacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bl, ahv, yacc[t], 0, 0, 0);
        }
      }
    }
    if (sb == SB - 1) {
      // row block done: logits out, running argmax, reset
      const int64_t nbase = (wave + k * n_waves) * 16 + 4 * g4;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t m = t * 16 + r;
        const v4f yv = yacc[t] * (1.0f / esc_t[t]);  // exact: a power of two
        if (m < M) {
          float* dst = p.logits + m * p.ldl + nbase;
          if (nbase + 3 < N && ((((uintptr_t)dst) & 15) == 0)) {
            __builtin_nontemporal_store(yv, (v4f*)dst);  // streamed out: its readers sit on other XCDs
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (nbase + i < N) dst[i] = yv[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t key = ((uint64_t)f32_order_bits(yv[i]) << 32) | (uint64_t)(~(uint32_t)(nbase + i));
          best[t] = (nbase + i < N && key > best[t]) ? key : best[t];
        }
        if (want_stats) {
          const float l[4] = {yv[0], yv[1], yv[2], yv[3]};
          const bool ok[4] = {nbase < N, nbase + 1 < N, nbase + 2 < N, nbase + 3 < N};
          softmax_add4(sm[t], ss[t], l, ok);
        }
        yacc[t] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
    advance(k, sb);
  };

  // three weight super-blocks in flight per wave: with two waves per SIMD
  // that is what covers the memory latency of this stream
  uint32_t rawA[RAWW], rawB[RAWW], rawC[RAWW];
  load_raw_dw<QT>(wr, woff(k2, sb2), g4, rawA);
  advance(k2, sb2);
  load_raw_dw<QT>(wr, woff(k2, sb2), g4, rawB);
  advance(k2, sb2);
  load_raw_dw<QT>(wr, woff(k2, sb2), g4, rawC);
  advance(k2, sb2);
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  int64_t st = 0;
  if constexpr (PARITY) {
    // step st has sb of the parity of st; six steps per iteration cover both
    // parities on all three buffers
    for (; st + 5 < n_steps; st += 6) {
      step(P1{}, rawA);
      step(P2{}, rawB);
      step(P1{}, rawC);
      step(P2{}, rawA);
      step(P1{}, rawB);
      step(P2{}, rawC);
    }
    if (st < n_steps) step(P1{}, rawA);
    if (st + 1 < n_steps) step(P2{}, rawB);
    if (st + 2 < n_steps) step(P1{}, rawC);
    if (st + 3 < n_steps) step(P2{}, rawA);
    if (st + 4 < n_steps) step(P1{}, rawB);
  } else {
    for (; st + 2 < n_steps; st += 3) {
      step(P0{}, rawA);
      step(P0{}, rawB);
      step(P0{}, rawC);
    }
    if (st < n_steps) step(P0{}, rawA);
    if (st + 1 < n_steps) step(P0{}, rawB);
  }

  // per token: best key over the wave's rows (lanes of one token differ in g4)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint64_t b = best[t];
    const uint64_t o1 = __shfl_xor(b, 16);
    b = o1 > b ? o1 : b;
    const uint64_t o2 = __shfl_xor(b, 32);
    b = o2 > b ? o2 : b;
    const int64_t m = t * 16 + r;
    if (g4 == 0 && m < M) p.keys[wave * M + m] = b;
    if (want_stats) {
      softmax_merge_groups(sm[t], ss[t]);
      if (g4 == 0 && m < M) p.stats[wave * M + m] = float2{sm[t], ss[t]};
    }
  }
}

constexpr int LM_NW = 8;  // waves per work-group (two per SIMD)

int lmhead_stream_waves() { return 256 * LM_NW; }

bool lmhead_stream_fits(int64_t K, int64_t n_rows) { return n_rows <= LM_TOK && K <= 256 * LM_SBMAX; }

int64_t lmhead_stream_slots(int64_t N) {
  const int64_t wgs_needed = ((N + 15) / 16 + LM_NW - 1) / LM_NW;
  return (wgs_needed < 256 ? wgs_needed : 256) * LM_NW;
}

hipError_t launch_lmhead_stream(int qtype, const LmParams& p, hipStream_t s) {
  const int64_t n_rb = (p.N + 15) / 16;
  const int64_t wgs_needed = (n_rb + LM_NW - 1) / LM_NW;
  const unsigned grid = (unsigned)(wgs_needed < 256 ? wgs_needed : 256);
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL((k_lmhead_stream<QT_Q4K, LM_NW, false>), dim3(grid), dim3(64 * LM_NW), 0, s, p);
  else if (p.SB % 2 == 0)
    hipLaunchKernelGGL((k_lmhead_stream<QT_Q6K, LM_NW, true>), dim3(grid), dim3(64 * LM_NW), 0, s, p);
  else
    hipLaunchKernelGGL((k_lmhead_stream<QT_Q6K, LM_NW, false>), dim3(grid), dim3(64 * LM_NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace dllm
