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
// Work-group: NW = 4, 8 or 12 waves, each with RB = 1 or 2 blocks of 16
// weight rows, x up to 160 tokens (TB blocks of 16); the seven tile
// configurations are listed at launch_cfg.  Activations of one super-block are
// staged in LDS and shared by the waves; each wave unpacks only its own rows.
// The weight side of the minimum term, -dmin * m, is exact as two f16 halves
// for every f16 dmin up to 65504/63 (a 6-bit m times an 11-bit significand
// whose lowest bit is at least 2^-24, subnormals included).  K may be split
// across work-groups (grid.y): each writes its partial tile to a workspace
// slice, and the last of a tile's work-groups to finish sums the slices in
// split order (no second kernel).  One work-group's work is the device
// function qgemm_wg; k_qgemm runs it on its own grid, and k_qgemm_pair runs
// two GEMMs of the same activations (two four-wave plans) in one grid.
#include "common.hpp"
#include "kernels.hpp"
#include "unpack.hpp"

namespace dllm {

// NW waves per work-group, RB row blocks of 16 weight rows per wave: the tile
// is 16 * RB * NW rows x 16 * TB tokens.  Each B fragment read from LDS feeds
// 2 * RB MFMAs.
// Four-wave tiles of at most 80 tokens fit two work-groups per CU (two waves
// per SIMD, each with its own barrier); larger tiles run one per CU.
// ST = 2: the activation stage of the next super-block is loaded while this
// one is used (double buffer, one barrier per step); with one row block per
// wave the next block's weights are also unpacked during this one's MFMAs.
// ST = 1: one stage, loaded at the start of each step (two barriers per
// step); with 4 waves this fits two work-groups per CU whose waits the other
// one's work fills.
// The K-split sum of one output tile (rows row_base .. + ROWS, tokens m0 ..
// + TOK, clipped to N and M) in split order, plus the bias per row: slices
// [S][M][ldo] f32 at p.out (ldo = p.ldo, a multiple of 64) -> p.red_y.
// Deterministic and the same for every tile: acc = ((0 + P_0) + P_1) + ...,
// then + bias.  The slices are read device-coherently (other work-groups, on
// other XCDs, wrote them in this kernel).  y takes 16-byte stores where the
// group of four rows lies inside N and y's rows allow it.
template <int ROWS, int TOK, int NTH>
__device__ __forceinline__ void sum_split_tile(const GemmParams& p, int64_t row_base, int64_t m0, int S, int tid) {
  constexpr uint32_t kNone = 0x80000000u;  // an offset past the slices: reads zeros, no memory access
  const int64_t N = p.N, M = p.M, ldo = p.ldo;
  const rsrc_t wsr = make_rsrc(p.out, (int64_t)S * M * ldo * 4);
  const uint32_t slice = (uint32_t)(M * ldo * 4);
  float* y = p.red_y;
  const float* bias = p.red_bias;
  const bool yvec = (p.red_ldy % 4 == 0) && ((((uintptr_t)y) & 15) == 0);
  // each thread owns KI groups of four rows; their loads for SB slices at a
  // time are all in flight together
  constexpr int G = ROWS / 4, ITEMS = TOK * G, KI = (ITEMS + NTH - 1) / NTH;
  constexpr int SBAT = KI <= 5 ? 4 : 2;
  int64_t mk[KI], nk[KI];
  bool ok[KI];
  uint32_t ek[KI];
  v4f acc[KI];
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const int idx = tid + k * NTH;
    const int t = idx / G, g = idx - t * G;
    mk[k] = m0 + t;
    nk[k] = row_base + 4 * g;
    ok[k] = idx < ITEMS && mk[k] < M && nk[k] < N;
    ek[k] = ok[k] ? (uint32_t)((mk[k] * ldo + nk[k]) * 4) : 0u;
    acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  for (int s = 0; s < S; s += SBAT) {
    v4u v[SBAT][KI];
#pragma unroll
    for (int j = 0; j < SBAT; ++j)
#pragma unroll
      for (int k = 0; k < KI; ++k)
        v[j][k] = buf_ld128_dev(wsr, (ok[k] && s + j < S) ? ek[k] + (uint32_t)(s + j) * slice : kNone);
    // in split order; a slice past S adds +0, which leaves the sum unchanged
#pragma unroll
    for (int j = 0; j < SBAT; ++j)
#pragma unroll
      for (int k = 0; k < KI; ++k) acc[k] += __builtin_bit_cast(v4f, v[j][k]);
  }
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    if (!ok[k]) continue;
    const int64_t m = mk[k], n = nk[k];
    float* dst = y + m * p.red_ldy + n;
    v4f a = acc[k];
    if (n + 3 < N) {
      if (bias) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] += bias[n + i];
      }
      if (yvec) {
        __builtin_nontemporal_store(a, (v4f*)dst);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = a[i];
      }
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) dst[i] = bias ? a[i] + bias[n + i] : a[i];
    }
  }
}

// A buffer offset past every operand (they stay below 2 GiB): a load there
// reads zeros and makes no memory access.
constexpr uint32_t kNoLoad = 0x80000000u;

// The LDS a work-group of one tile configuration uses (sizes of its arrays).
//  * The activation stage: the int8 quants of TOKP tokens (TOK padded so the
//    buffer-to-LDS loads fill it exactly; the padding rows are loaded and
//    never read).  Two stages (double buffer) are separate objects: where each
//    step names them directly the compiler sees that the buffer-to-LDS loads
//    filling one stage do not alias the reads of the other, and does not wait
//    for those loads before the reads.  One stage (ST = 1) is the first
//    object, or with SPLIT both, tokens [0, H) in the first and the rest in
//    the second (so that both forms fit the same arrays in a grouped kernel).
//  * d_x staging: items (a token, or for Q4_K a (token, half q) pair that
//    covers sub-blocks 4q .. 4q+3) are spread over the loading threads.
//    Token t's d_x sits at slot t (written by its item with q = 0); every
//    other item writes a slot of its own past TOK, which nothing reads, so
//    every store is unconditional and has its own address.  DXS floats per
//    stage.
//  * Q4_K: an 8-slot ring (two groups of four super-blocks) of min-term
//    activation operands, high halves [slot][token][8] f16 then low halves
//    likewise: one group is read while the next is written.  A lane's 16-byte
//    read of one token's eight values has consecutive tokens at consecutive
//    16-byte slots, so the reads of a wave hit distinct banks.
//  * the per-token pre-scale, and the argmax epilogue's keys and statistics.
template <int QT, int TB, int NW, int RB, bool ARGMAX, int ST, bool SPLIT = false>
struct QgemmLds {
  static constexpr bool ONE = (ST == 1);
  static constexpr bool MINS = (QT == QT_Q4K);
  static constexpr int TOK = TB * 16;  // tokens per work-group (MFMA columns)
  // Stage loads and d_x items are issued by the first LW waves only: with
  // two or more waves per SIMD the others then start each step on the matrix
  // cores instead of queueing behind the first ones' loads.
  static constexpr int LW = (!ONE && RB == 1 && NW >= 8) ? 4 : NW;
  static constexpr int TOKP = (TOK + 4 * LW - 1) / (4 * LW) * (4 * LW);
  static constexpr int H = (ONE && SPLIT) ? 16 * ((TB + 1) / 2) : TOKP;
  static constexpr int ACT0 = H * ACT_ROW;
  static constexpr int ACT1 = ONE ? (TOKP > H ? (TOKP - H) * ACT_ROW : 16) : TOKP * ACT_ROW;
  static constexpr bool SPLIT1 = ONE && TOKP > H;  // the one stage spans both arrays
  static constexpr int NTHL = 64 * LW;
  static constexpr int NITEM = MINS ? TOK * 2 : TOK;
  static constexpr int IPT = (NITEM + NTHL - 1) / NTHL;  // items per loading thread
  static constexpr int DXS = TOK + IPT * NTHL;
  static constexpr int DX = (ONE ? 1 : 2) * DXS;
  static constexpr int AMS = 8;                    // halves per token record of the ring
  static constexpr int RSLOTS = ONE ? 4 : 8;       // ring slots (one group, or two)
  static constexpr int AMLO = RSLOTS * TOK * AMS;  // offset of the low halves
  static constexpr int AMIN = MINS ? 2 * AMLO + 8 * (IPT * NTHL - NITEM) + 8 : 8;
  static constexpr int KEYS = ARGMAX ? NW * TOK : 1;
};

// The LDS arrays of a work-group (at least the QgemmLds sizes), given by the
// kernel that declares them.
struct QgemmSmem {
  uint8_t* act0;
  uint8_t* act1;
  float* dx;
  float* esc;
  _Float16* amin;
  uint64_t* key;
  float2* stat;
  int* last;
};

// Which tile a work-group computes: (bx, by, bz) of a (gx, gy, *) grid of
// row tiles, K splits and token tiles.  HwTile: the work-group's own place in
// its grid; WgTile: a place given by the kernel.
struct HwTile {
  __device__ uint32_t bx() const { return blockIdx.x; }
  __device__ uint32_t by() const { return blockIdx.y; }
  __device__ uint32_t bz() const { return blockIdx.z; }
  __device__ uint32_t gx() const { return gridDim.x; }
  __device__ uint32_t gy() const { return gridDim.y; }
};
struct WgTile {
  uint32_t x, y, z, nx, ny;
  __device__ uint32_t bx() const { return x; }
  __device__ uint32_t by() const { return y; }
  __device__ uint32_t bz() const { return z; }
  __device__ uint32_t gx() const { return nx; }
  __device__ uint32_t gy() const { return ny; }
};

// One work-group of the GEMM: tile t.
// SUMS: the test form, which also stores every tile's exact int32
// super-block sums A_sb = (hi << shift) + lo, as formed for the epilogue, to
// ((int32_t*)p.out)[(m * N + n) * SB + sb], and writes no y.
template <int QT, int TB, int NW, int RB, bool ARGMAX, int ST, bool SUMS, bool SPLIT, class TILE>
__device__ __forceinline__ void qgemm_wg(const GemmParams p, const TILE wt, const QgemmSmem lds) {
  static_assert(NW == 4 || NW == 8 || NW == 12, "waves per work-group: 4, 8 or 12 (whole SIMDs)");
  static_assert(ST == 2 || NW == 4, "one activation stage: four waves");
  using G = QgemmLds<QT, TB, NW, RB, ARGMAX, ST, SPLIT>;
  constexpr bool ONE = (ST == 1);
  constexpr int TOK = G::TOK;
  constexpr int NTH = 64 * NW;          // threads
  constexpr int ROWS = 16 * RB * NW;    // weight rows per work-group
  constexpr int SHIFT = QTr<QT>::SHIFT;
  constexpr int BYTES = QTr<QT>::BYTES;
  constexpr int RAW = QTr<QT>::RAW;
  constexpr bool MINS = G::MINS;
  constexpr int LW = G::LW;
  constexpr int NTHL = G::NTHL;
  // buffer-to-LDS loads per loading wave per stage: 16 units per token, 64
  // units per wave-wide load
  constexpr int DPW = G::TOKP * 16 / (64 * LW);
  constexpr int AMS = G::AMS;
  constexpr int AMLO = G::AMLO;
  constexpr int NITEM = G::NITEM;
  constexpr int IPT = G::IPT;
  constexpr int DXS = G::DXS;
  uint8_t* const s_act0 = lds.act0;
  uint8_t* const s_act1 = lds.act1;
  float* const s_dx = lds.dx;
  float* const s_esc = lds.esc;
  _Float16* const s_amin = lds.amin;
  uint64_t* const s_key = lds.key;
  float2* const s_stat = lds.stat;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t N = p.N, SB = p.SB, M = p.M;
  const int64_t m0 = (int64_t)wt.bz() * TOK;
  const int64_t s0 = (int64_t)wt.by() * p.sps;
  const int64_t s1 = (s0 + p.sps < SB) ? s0 + p.sps : SB;
  const int64_t row0 = (int64_t)wt.bx() * ROWS + wv * 16 * RB;  // first row of this wave
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

  // SUMS: a lane's integer tile sums are rows row0 + 16 b + 4 g4 + i of
  // token m0 + 16 t + r
  auto sums_store = [&](int t, int b, int64_t sb, const v4i& al, const v4i& ah) {
    if constexpr (SUMS) {
      const int64_t m = m0 + t * 16 + r;
      const int64_t nb = row0 + 16 * b + 4 * g4;
      int32_t* P = (int32_t*)p.out;
      if (m < M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nb + i < N) P[(m * N + nb + i) * SB + sb] = (ah[i] << SHIFT) + al[i];
      }
    }
  };

  // ---- activation staging.  The int8 quants go global -> LDS directly:
  // load k of wave wv fills LDS units (wv DPW + k) 64 + lane, i.e. token
  // u >> 4, slot u & 15, with global unit (slot ^ token) of that token's
  // record (its quants start 4 bytes in).  d_x (and for Q4_K the min-term
  // operands, one (token, j) pair per item) go through registers.  Every load
  // is unconditional -- past the end of the operand the buffer reads zero --
  // and so is every store (to its own LDS address).
  const uint32_t dma_tok0 = (uint32_t)((m0 + wv * DPW * 4 + (lane >> 4)) * SB * Q8K_BYTES) + 4;
  const uint32_t tok_step = (uint32_t)(4 * SB * Q8K_BYTES);
  auto act_dma = [&](uint8_t* stage, int64_t sb) {
    if constexpr (LW < NW) {
      if (wv >= LW) return;
    }
    const uint32_t soff = (uint32_t)(sb * Q8K_BYTES);
#pragma unroll
    for (int k = 0; k < DPW; ++k) {
      const int j = wv * DPW + k;  // LDS units 64 j .. 64 j + 63: tokens 4 j .. 4 j + 3
      const int tok = j * 4 + (lane >> 4);
      const uint32_t voff = dma_tok0 + k * tok_step + 16 * ((lane & 15) ^ (tok & 15));
      uint8_t* dst;
      if constexpr (G::SPLIT1) dst = (4 * j < G::H) ? s_act0 + j * 1024 : s_act1 + (j - G::H / 4) * 1024;
      else if constexpr (ONE) dst = s_act0 + j * 1024;
      else dst = stage + j * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0,
                                               0);
    }
  };
  // idx_b: Q4_K bsum pairs (2j, 2j+1) for j = 4q .. 4q+3, one per dword
  uint32_t idx_d[IPT];
  v4u idx_b[MINS ? IPT : 1];
  auto items_load = [&](int64_t sb) {
    if constexpr (LW < NW) {
      if (wv >= LW) return;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int item = tid + k * NTHL;
      const int it_c = item < NITEM ? item : NITEM - 1;
      const int tok = MINS ? (it_c >> 1) : it_c;
      const uint32_t xoff = (uint32_t)(((m0 + tok) * SB + sb) * Q8K_BYTES);
      idx_d[k] = buf_ld32(xr, xoff);
      if constexpr (MINS) idx_b[k] = buf_ld128(xr, xoff + 260 + 16 * (it_c & 1));
    }
  };
  auto items_store = [&](int buf, int slot8) {
    if constexpr (LW < NW) {
      if (wv >= LW) return;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int item = tid + k * NTHL;
      const bool live = item < NITEM;
      const int it_c = live ? item : NITEM - 1;
      const int tok = MINS ? (it_c >> 1) : it_c;
      const float dx = __builtin_bit_cast(float, idx_d[k]) * s_esc[tok];
      if constexpr (!MINS) s_dx[buf * DXS + item] = dx;
      if constexpr (MINS) {
        const int q = it_c & 1;
        s_dx[buf * DXS + ((live && q == 0) ? tok : TOK + item)] = dx;
        // activation side of the min term: d_x * (bsum_{2j} + bsum_{2j+1})
        // for j = 4q .. 4q+3, as f16 high and low halves
        typedef _Float16 v4h __attribute__((ext_vector_type(4)));
        v4h hv, lv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t pr = idx_b[k][i];
          const int S = (int)(int16_t)(pr & 0xFFFFu) + (int)(int16_t)(pr >> 16);
          _Float16 h, l;
          split_f16(dx * (float)S, h, l);
          hv[i] = h;
          lv[i] = l;
        }
        _Float16* dm_hi = s_amin + (live ? (slot8 * TOK + tok) * AMS + 4 * q : 2 * AMLO + 8 * (item - NITEM));
        _Float16* dm_lo = live ? dm_hi + AMLO : dm_hi + 4;
        *(v4h*)dm_hi = hv;
        *(v4h*)dm_lo = lv;
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

  // One super-block: start the next stage's loads, unpack this block's
  // weights (loaded during the previous step into `raw`, which is then
  // refilled with the next block), contract on MFMA, fold in the min term at
  // the end of a group of four, publish the next stage's d_x.  The barrier at
  // the end also waits for every load in flight.
  uint32_t raw[RB][RAW];
  // act: this step's stage; act_next: the other one, filled for sb + 1;
  // buf == (sb - s0) & 1 indexes the d_x stages.
  auto step = [&](int64_t sb, const uint8_t* act, uint8_t* act_next, int buf) {
    const int it = (int)(sb - s0);
    const int slot = it & 3;
    const bool more = sb + 1 < s1;
    if constexpr (ONE) {
      act_dma(nullptr, sb);
      items_load(sb);
    } else {
      act_dma(act_next, sb + 1);  // past the end: an unread stage
      items_load(sb + 1);
    }
    v4i alo[RB][4], ahi[RB][4];
    float dsel[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const uint32_t boff = wrow_off[b] + (uint32_t)(sb * BYTES);
      const float drow = unpack<QT>(raw[b], g4, alo[b], ahi[b]);
      if constexpr (MINS) {
        const bool mine = (slot == g4);
        mh0[b] = mine ? raw[b][0] : mh0[b];
        mh2[b] = mine ? raw[b][2] : mh2[b];
        mh3[b] = mine ? raw[b][3] : mh3[b];
      }
      if constexpr (!ONE) load_raw<QT>(wr, boff + BYTES, g4, raw[b]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dsel[b][i] = __shfl(drow, 4 * g4 + i);
    }
    if constexpr (ONE) {
      // publish this step's d_x and min-term operands; the barrier also
      // waits for the stage loads.  The next weights are requested after it,
      // so that the wait does not include them.
      items_store(0, slot);
      __syncthreads();
#pragma unroll
      for (int b = 0; b < RB; ++b) load_raw<QT>(wr, wrow_off[b] + (uint32_t)((sb + 1) * BYTES), g4, raw[b]);
    }

    // integer contraction (two planes x four K chunks x RB row blocks) and
    // the super-block epilogue y += (d * d_x) * ((hi << shift) + lo),
    // software-pipelined: the B fragments of token block t+1 are read while
    // block t's MFMAs run, and each (token block, row block) tile's integer
    // sums are folded into y while the next tile's MFMAs run.
    int bunit[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bunit[c] = 16 * (act_unit<QT>(c, g4) ^ r);  // token t*16 + r has (tok & 15) == r
    auto loadB = [&](int t, v4i(&dstB)[4]) {
      const uint8_t* arow;
      if constexpr (G::SPLIT1)
        arow = (t * 16 < G::H) ? s_act0 + (t * 16 + r) * ACT_ROW : s_act1 + (t * 16 - G::H + r) * ACT_ROW;
      else if constexpr (ONE) arow = s_act0 + (t * 16 + r) * ACT_ROW;
      else arow = act + (t * 16 + r) * ACT_ROW;
#pragma unroll
      for (int c = 0; c < 4; ++c) dstB[c] = *(const v4i*)(arow + bunit[c]);
    };
    auto flush = [&](int t, int b, const v4i& al, const v4i& ah) {
      sums_store(t, b, sb, al, ah);
      const float dx = s_dx[buf * DXS + t * 16 + r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = (ah[i] << SHIFT) + al[i];
        yacc[b][t][i] = __builtin_fmaf((float)a, dsel[b][i] * dx, yacc[b][t][i]);
      }
    };
    v4i Bc[4], Bn[4];
    loadB(0, Bc);
    v4i pl = {0, 0, 0, 0}, ph = {0, 0, 0, 0};  // the tile waiting to be folded in
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t + 1 < TB) loadB(t + 1, Bn);
      // keep the next block's fragment reads ahead of this block's MFMAs (the
      // scheduler would otherwise sink each read next to its use and expose
      // the LDS latency)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        v4i al = {0, 0, 0, 0}, ah = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          al = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[b][c], Bc[c], al, 0, 0, 0);
          ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi[b][c], Bc[c], ah, 0, 0, 0);
        }
        if (b > 0) flush(t, b - 1, pl, ph);
        else if (t > 0) flush(t - 1, RB - 1, pl, ph);
        pl = al;
        ph = ah;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) Bc[c] = Bn[c];
      __builtin_amdgcn_sched_barrier(0);
    }
    flush(TB - 1, RB - 1, pl, ph);

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
        const int gbase = ONE ? 0 : (it & 4);  // ring slots of this group: gbase .. gbase + 3
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const _Float16* src = s_amin + ((gbase + g4) * TOK + t * 16 + r) * AMS;
          const v8h ahv = *(const v8h*)src;
          const v8h alv = *(const v8h*)(src + AMLO);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            yacc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_hi[b], ahv, yacc[b][t], 0, 0, 0);
            yacc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_hi[b], alv, yacc[b][t], 0, 0, 0);
            yacc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_lo[b], ahv, yacc[b][t], 0, 0, 0);
          }
        }
      }
    }
    if constexpr (ONE) {
      __syncthreads();  // every read of the stage done before the next fill
    } else {
      items_store(buf ^ 1, (it + 1) & 7);  // past the end: an unread stage
      __syncthreads();
    }
  };

  // Pipelined form (two stages, one row block per wave): the weights of the
  // step's block were unpacked during the previous step; the next block's
  // unpack runs chunk by chunk between this block's token tiles, where its
  // VALU work issues beside the MFMAs, and its raw data is then refilled
  // with the block after it.
  struct AState {
    v4i lo[4], hi[4];
    float dsel[4];
  };
  AState A0, A1;
  uint32_t mhn0 = 0u, mhn2 = 0u, mhn3 = 0u;
  auto unpack_full = [&](AState& A) {
    const float drow = unpack<QT>(raw[0], g4, A.lo, A.hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) A.dsel[i] = __shfl(drow, 4 * g4 + i);
  };
  auto step_pp = [&](int64_t sb, const uint8_t* act, uint8_t* act_next, int buf, AState& A, AState& An) {
    const int it = (int)(sb - s0);
    const int slot = it & 3;
    const bool more = sb + 1 < s1;
    act_dma(act_next, sb + 1);  // past the end: an unread stage
    items_load(sb + 1);
    // the block after next, which raw is refilled with once the next one is
    // unpacked; past the split's end an offset beyond the buffer, which reads
    // zeros without touching memory (the load is issued either way, so the
    // waits stay the same on every path)
    const uint32_t noff = (sb + 2 < s1) ? wrow_off[0] + (uint32_t)((sb + 2) * BYTES) : kNoLoad;
    uint32_t sc03 = 0u, sc47 = 0u, mn03, mn47;
    if constexpr (MINS) {
      q4k_scales(raw[0][1], raw[0][2], raw[0][3], sc03, sc47, mn03, mn47);
      mhn0 = raw[0][0];
      mhn2 = raw[0][2];
      mhn3 = raw[0][3];
    }
    const float dnext = f16_bits_to_f32(MINS ? raw[0][0] : raw[0][RAW - 1]);
    int bunit[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bunit[c] = 16 * (act_unit<QT>(c, g4) ^ r);
    auto loadB = [&](int t, v4i(&dstB)[4]) {
      const uint8_t* arow = act + (t * 16 + r) * ACT_ROW;
#pragma unroll
      for (int c = 0; c < 4; ++c) dstB[c] = *(const v4i*)(arow + bunit[c]);
    };
    float dxr[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) dxr[t] = s_dx[buf * DXS + t * 16 + r];
    auto flush = [&](int t, const v4i& al, const v4i& ah) {
      sums_store(t, 0, sb, al, ah);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = (ah[i] << SHIFT) + al[i];
        yacc[0][t][i] = __builtin_fmaf((float)a, A.dsel[i] * dxr[t], yacc[0][t][i]);
      }
      asm volatile("" : "+v"(yacc[0][t]));
    };
    // with three waves per SIMD the others hide a tile's fragment reads, and
    // the registers of a second fragment set are not there
    constexpr bool BPRE = (NW < 12);
    v4i Bc[4], Bn[4];
    if constexpr (BPRE) loadB(0, Bc);
    // the matrix loop runs at a raised wave priority, so that waves in it win
    // issue slots over waves doing staging work
    __builtin_amdgcn_s_setprio(1);
    v4i pl = {0, 0, 0, 0}, ph = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if constexpr (BPRE) {
        if (t + 1 < TB) loadB(t + 1, Bn);
      } else {
        loadB(t, Bc);
      }
      __builtin_amdgcn_sched_barrier(0);
      v4i al = {0, 0, 0, 0}, ah = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        al = __builtin_amdgcn_mfma_i32_16x16x64_i8(A.lo[c], Bc[c], al, 0, 0, 0);
        ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(A.hi[c], Bc[c], ah, 0, 0, 0);
      }
      if (t > 0) flush(t - 1, pl, ph);
      pl = al;
      ph = ah;
      // the next block's chunks, spread over the tiles
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((c * TB) / 4 == t) {
          unpack_chunk<QT>(raw[0], g4, c, sc03, sc47, An.lo[c], An.hi[c]);
          // pinned here (with four waves, which have the registers):
          // otherwise the compiler sinks the unpack to the next step, where
          // it runs as one burst ahead of that step's first MFMA
          if constexpr (NW == 4) asm volatile("" : "+v"(An.lo[c]), "+v"(An.hi[c]));
        }
      if (t == (3 * TB) / 4) load_raw<QT>(wr, noff, g4, raw[0]);
      if (t == TB - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) An.dsel[i] = __shfl(dnext, 4 * g4 + i);
      }
      if constexpr (BPRE) {
#pragma unroll
        for (int c = 0; c < 4; ++c) Bc[c] = Bn[c];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    flush(TB - 1, pl, ph);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (MINS) {
      if (slot == 3 || !more) {
        v8h bmin_hi, bmin_lo;
        const bool live = row_ok[0] && g4 <= slot;
        uint32_t q03, q47, mn03, mn47;
        q4k_scales(0u, live ? mh2[0] : 0u, live ? mh3[0] : 0u, q03, q47, mn03, mn47);
        const float ndmin = -f16_bits_to_f32(live ? (mh0[0] >> 16) : 0u);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t mb = (j < 4) ? mn03 : mn47;
          _Float16 hi, lo;
          split_f16(ndmin * (float)((mb >> (8 * (j & 3))) & 63u), hi, lo);
          bmin_hi[j] = hi;
          bmin_lo[j] = lo;
        }
        const int gbase = it & 4;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const _Float16* src = s_amin + ((gbase + g4) * TOK + t * 16 + r) * AMS;
          const v8h ahv = *(const v8h*)src;
          const v8h alv = *(const v8h*)(src + AMLO);
          yacc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_hi, ahv, yacc[0][t], 0, 0, 0);
          yacc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_hi, alv, yacc[0][t], 0, 0, 0);
          yacc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bmin_lo, ahv, yacc[0][t], 0, 0, 0);
        }
      }
      // the next block's min-term bytes, now that this group's are used
      const bool mine = (((it + 1) & 3) == g4);
      mh0[0] = mine ? mhn0 : mh0[0];
      mh2[0] = mine ? mhn2 : mh2[0];
      mh3[0] = mine ? mhn3 : mh3[0];
    }
    items_store(buf ^ 1, (it + 1) & 7);  // past the end: an unread stage
    __syncthreads();
  };

  // ---- prologue: the first weights and activation stage are requested
  // first, so that their latency overlaps the pre-scale scan below.
#pragma unroll
  for (int b = 0; b < RB; ++b) load_raw<QT>(wr, wrow_off[b] + (uint32_t)(s0 * BYTES), g4, raw[b]);
  if constexpr (!ONE) {
    act_dma(s_act0, s0);
    items_load(s0);
  }


  // Per-token power-of-two pre-scale of d_x (Q4_K: keeps the f16 halves of
  // d_x * S_j in range; undone exactly at the end); 1 for Q6_K.  It comes
  // from the token's largest |d| over the whole row: given by the caller, or
  // else found by reading every block's d (one cache line per block).
  if (tid < TOK) {
    float esc = 1.0f;
    if constexpr (MINS) {
      float mx = 0.0f;
      if (p.dmax) {
        if (m0 + tid < M) mx = p.dmax[m0 + tid];
      } else {
        // sixteen independent loads in flight per round
        const uint32_t tok_off = (uint32_t)((m0 + tid) * SB * Q8K_BYTES);
        for (int64_t sb = 0; sb < SB; sb += 16) {
          float v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) v[u] = __builtin_bit_cast(float, buf_ld32(xr, tok_off + (uint32_t)((sb + u) * Q8K_BYTES)));
#pragma unroll
          for (int u = 0; u < 16; ++u) mx = (sb + u < SB) ? fmaxf(mx, __builtin_fabsf(v[u])) : mx;
        }
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
    for (int i = tid; i < 2 * AMLO / 8; i += NTH) ((v4u*)s_amin)[i] = v4u{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if constexpr (!ONE) {
    items_store(0, 0);
    __syncthreads();
  }

  if constexpr (ONE) {
    for (int64_t sb = s0; sb < s1; ++sb) step(sb, nullptr, nullptr, 0);
  } else if constexpr (RB == 1) {
    // the first block is unpacked here (and its min-term bytes kept); then
    // two steps per iteration, each naming its stages and weights directly
    unpack_full(A0);
    if constexpr (MINS) {
      const bool mine = (g4 == 0);
      mh0[0] = mine ? raw[0][0] : 0u;
      mh2[0] = mine ? raw[0][2] : 0u;
      mh3[0] = mine ? raw[0][3] : 0u;
    }
    load_raw<QT>(wr, s0 + 1 < s1 ? wrow_off[0] + (uint32_t)((s0 + 1) * BYTES) : kNoLoad, g4, raw[0]);
    int64_t sb = s0;
    for (; sb + 1 < s1; sb += 2) {
      step_pp(sb, s_act0, s_act1, 0, A0, A1);
      step_pp(sb + 1, s_act1, s_act0, 1, A1, A0);
    }
    if (sb < s1) step_pp(sb, s_act0, s_act1, 0, A0, A1);
  } else {
    // one step per iteration (fewer live registers; the compiler then waits
    // for the stage loads before the step's first LDS read)
    for (int64_t sb = s0; sb < s1; ++sb) {
      const int buf = (int)(sb - s0) & 1;
      step(sb, buf ? s_act1 : s_act0, buf ? s_act0 : s_act1, buf);
    }
  }

  // ---- write out: lane holds rows nbase + i (i < 4) of token t*16 + r
  // (plus the bias of those rows, when given: only without a K split, whose
  // reduction adds it instead)
  if constexpr (SUMS) return;
  float* outp = p.out + (int64_t)wt.by() * p.split_stride;
  // K split with the reduction fused: the slice [M][ldo] goes out with
  // device-coherent 16-byte stores (ldo a multiple of 64 >= N, so every
  // group of four rows that starts inside N is whole)
  const rsrc_t wsr = make_rsrc(p.out, p.tile_cnt ? (int64_t)wt.gy() * p.split_stride * 4 : 0);
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int64_t nbase = row0 + 16 * b + 4 * g4;
    v4f bv = {0.f, 0.f, 0.f, 0.f};
    if (p.bias) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nbase + i < N) bv[i] = p.bias[nbase + i];
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int64_t m = m0 + t * 16 + r;
      const float inv = 1.0f / s_esc[t * 16 + r];  // exact: a power of two
      const v4f yv = p.bias ? yacc[b][t] * inv + bv : yacc[b][t] * inv;
      yacc[b][t] = yv;
      if (p.tile_cnt) {
        if (m < M && nbase < N)
          buf_st128_dev(wsr, (uint32_t)(((int64_t)wt.by() * p.split_stride + m * p.ldo + nbase) * 4),
                        __builtin_bit_cast(v4u, yv));
      } else if (m < M) {
        float* dst = outp + m * p.ldo + nbase;
        if (nbase + 3 < N && ((((uintptr_t)dst) & 15) == 0)) {
          // streamed out (non-temporal): the readers of y or of the split
          // partials run on other XCDs and read them from memory anyway, and
          // no dirty lines are left in this XCD's L2 for the kernel's end
          __builtin_nontemporal_store(yv, (v4f*)dst);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nbase + i < N) dst[i] = yv[i];
        }
      }
    }
  }

  if (p.tile_cnt) {
    // K split with the reduction fused: once this work-group's slice has
    // reached memory (each wave waits for its own stores), it is counted in
    // with a device-scope atomic; the last of the tile's gy
    // work-groups to arrive sums the slices.  That last arrival also resets
    // the counter, so the next call on the stream finds it 0.  The slices
    // are written and read with device-coherent accesses, so no cache
    // maintenance is needed on either side.
    int* const s_last = lds.last;
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      uint32_t* c = p.tile_cnt + (int64_t)wt.bz() * wt.gx() + wt.bx();
      const uint32_t before = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = (before + 1 == wt.gy());
      if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = last ? 1 : 0;
    }
    __syncthreads();
    if (*s_last) sum_split_tile<ROWS, TOK, NTH>(p, (int64_t)wt.bx() * ROWS, m0, (int)wt.gy(), tid);
  }

  if constexpr (ARGMAX) {
    // per token: best (value, lowest row index) over this work-group's rows
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      // every key is formed and rows past N select 0 (no branch per element)
      uint64_t best = 0;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t n = row0 + 16 * b + 4 * g4 + i;
          const uint64_t key = ((uint64_t)f32_order_bits(yacc[b][t][i]) << 32) | (uint64_t)(~(uint32_t)n);
          const uint64_t kv = n < N ? key : 0ull;
          best = kv > best ? kv : best;
        }
      const uint64_t o1 = __shfl_xor(best, 16);
      best = o1 > best ? o1 : best;
      const uint64_t o2 = __shfl_xor(best, 32);
      best = o2 > best ? o2 : best;
      if (g4 == 0) s_key[wv * TOK + t * 16 + r] = best;
      if (p.stats) {
        // softmax statistics of this token over the wave's rows
        float sm = -__builtin_inff(), ss = 0.0f;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const float l[4] = {yacc[b][t][0], yacc[b][t][1], yacc[b][t][2], yacc[b][t][3]};
          bool ok[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ok[i] = row0 + 16 * b + 4 * g4 + i < N;
          softmax_add4(sm, ss, l, ok);
        }
        softmax_merge_groups(sm, ss);
        if (g4 == 0) s_stat[wv * TOK + t * 16 + r] = float2{sm, ss};
      }
    }
    __syncthreads();
    if (tid < TOK) {
      const int64_t m = m0 + tid;
      uint64_t best = s_key[tid];
#pragma unroll
      for (int k = 1; k < NW; ++k) best = s_key[k * TOK + tid] > best ? s_key[k * TOK + tid] : best;
      if (m < M) p.keys[(int64_t)wt.bx() * M + m] = best;
      if (p.stats) {
        float sm = s_stat[tid].x, ss = s_stat[tid].y;
#pragma unroll
        for (int k = 1; k < NW; ++k) softmax_merge(sm, ss, s_stat[k * TOK + tid].x, s_stat[k * TOK + tid].y);
        if (m < M) p.stats[(int64_t)wt.bx() * M + m] = float2{sm, ss};
      }
    }
  }
}

// The LDS arrays of a kernel: one set per instantiation of the sizes (the
// largest of its configurations' for a kernel that runs several).
template <int A0, int A1, int DX, int ESC, int AMIN, int KEYS>
__device__ __forceinline__ QgemmSmem qgemm_lds() {
  __shared__ __attribute__((aligned(16))) uint8_t s_act0[A0];
  __shared__ __attribute__((aligned(16))) uint8_t s_act1[A1];
  __shared__ float s_dx[DX];
  __shared__ float s_esc[ESC];
  __shared__ __attribute__((aligned(16))) _Float16 s_amin[AMIN];
  __shared__ uint64_t s_key[KEYS];
  __shared__ float2 s_stat[KEYS];
  __shared__ int s_last;
  return QgemmSmem{s_act0, s_act1, s_dx, s_esc, s_amin, s_key, s_stat, &s_last};
}

template <int QT, int TB, int NW, int RB, bool ARGMAX, int ST = 2, bool SUMS = false>
__global__ __launch_bounds__(64 * NW, (NW == 4 && (TB <= 5 || ST == 1)) ? 2 : 1) void k_qgemm(GemmParams p) {
  using G = QgemmLds<QT, TB, NW, RB, ARGMAX, ST>;
  const QgemmSmem lds = qgemm_lds<G::ACT0, G::ACT1, G::DX, G::TOK, G::AMIN, G::KEYS>();
  qgemm_wg<QT, TB, NW, RB, ARGMAX, ST, SUMS, false>(p, HwTile{}, lds);
}

// Two GEMMs over the same activations in one launch (a grouped launch): the
// work-groups of A's grid and of B's grid, both four-wave tiles that fit two
// work-groups per CU, share one grid, so that a CU holds a work-group of each
// where either launch alone would leave it half used.  Blocks go in groups
// of eight (one per XCD, in dispatch order), alternating A and B while both
// have groups left; a work-group's index in its own grid keeps its place
// modulo 8, so each tile runs on the XCD it would have run on alone.  Every
// tile computes exactly what it computes in its own launch.
struct PairGrid {
  int64_t n[2];       // work-groups of A's and B's grid
  int64_t gx[2], gy[2];
  int64_t groups[2];  // groups of eight blocks: cdiv(n, 8)
};

template <int Q, int TB, int ST>
struct Cfg4 {  // a four-wave, one-row-block tile configuration (one stage split over both arrays)
  static constexpr int QT = Q, T = TB, S = ST;
  using G = QgemmLds<Q, TB, 4, 1, false, ST, true>;
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <class CA, class CB>
__global__ __launch_bounds__(256, 2) void k_qgemm_pair(GemmParams pa, GemmParams pb, PairGrid g) {
  using GA = typename CA::G;
  using GB = typename CB::G;
  const QgemmSmem lds = qgemm_lds<cmax(GA::ACT0, GB::ACT0), cmax(GA::ACT1, GB::ACT1), cmax(GA::DX, GB::DX),
                                  cmax(GA::TOK, GB::TOK), cmax(GA::AMIN, GB::AMIN), 1>();
  const int64_t grp = blockIdx.x >> 3, k = blockIdx.x & 7;
  const int64_t both = g.groups[0] < g.groups[1] ? g.groups[0] : g.groups[1];
  int which;
  int64_t gi;
  if (grp < 2 * both) {
    which = (int)(grp & 1);
    gi = grp >> 1;
  } else {
    which = g.groups[0] > g.groups[1] ? 0 : 1;
    gi = grp - both;
  }
  const int64_t li = gi * 8 + k;  // index in that GEMM's own grid
  if (li >= g.n[which]) return;   // the tail of a partial group (whole work-group)
  const int64_t gx = g.gx[which], gy = g.gy[which];
  const int64_t rest = li / gx;
  const WgTile wt{(uint32_t)(li - rest * gx), (uint32_t)(rest % gy), (uint32_t)(rest / gy), (uint32_t)gx,
                  (uint32_t)gy};
  if (which == 0) qgemm_wg<CA::QT, CA::T, 4, 1, false, CA::S, false, true>(pa, wt, lds);
  else qgemm_wg<CB::QT, CB::T, 4, 1, false, CB::S, false, true>(pb, wt, lds);
}

// argmax[m] = lowest row index of the largest logit, from per-tile keys.
// With stats, also the row's log-sum-exp and the softmax probability of its
// largest logit, from the per-tile (m, s) statistics merged in a tree.
__global__ __launch_bounds__(256) void k_argmax_finalize(const uint64_t* __restrict__ keys,
                                                       const float2* __restrict__ stats, int64_t n_tiles,
                                                       int64_t M, int32_t* __restrict__ argmax,
                                                       float* __restrict__ lse, float* __restrict__ p_max) {
  __shared__ uint64_t red[256];
  __shared__ float2 sred[256];
  const int64_t m = blockIdx.x;
  uint64_t best = 0;
  float sm = -__builtin_inff(), ss = 0.0f;
  for (int64_t t = threadIdx.x; t < n_tiles; t += 256) {
    const uint64_t k = keys[t * M + m];
    best = k > best ? k : best;
    if (stats) {
      const float2 st = stats[t * M + m];
      softmax_merge(sm, ss, st.x, st.y);
    }
  }
  red[threadIdx.x] = best;
  sred[threadIdx.x] = float2{sm, ss};
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      if (red[threadIdx.x + s] > red[threadIdx.x]) red[threadIdx.x] = red[threadIdx.x + s];
      if (stats) {
        float a = sred[threadIdx.x].x, b = sred[threadIdx.x].y;
        softmax_merge(a, b, sred[threadIdx.x + s].x, sred[threadIdx.x + s].y);
        sred[threadIdx.x] = float2{a, b};
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    argmax[m] = (int32_t)(~(uint32_t)(red[0] & 0xFFFFFFFFu));
    if (stats) {
      lse[m] = sred[0].x + logf(sred[0].y);
      p_max[m] = 1.0f / sred[0].y;
    }
  }
}

// Test export: per-16 integer partial dots of the unsigned shared-form quants
// with the Q8_K quants, with the quants taken from the GGUF bit layout by the
// shared nibble and field helpers (the GEMM's fragment unpacking produces the
// same quants in its own K order).
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
template <int QT, int TB, int NW, int RB, bool ARGMAX, int ST = 2, bool SUMS = false>
static hipError_t launch_k(const GemmParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_qgemm<QT, TB, NW, RB, ARGMAX, ST, SUMS>), grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

template <int QT, int NW, int RB, bool ARGMAX, int ST = 2>
static hipError_t launch_q(const GemmParams& p, int tb, dim3 grid, hipStream_t s) {
  switch (tb) {
    case 1: return launch_k<QT, 1, NW, RB, ARGMAX, ST>(p, grid, s);
    case 2: return launch_k<QT, 2, NW, RB, ARGMAX, ST>(p, grid, s);
    case 3: return launch_k<QT, 3, NW, RB, ARGMAX, ST>(p, grid, s);
    case 4: return launch_k<QT, 4, NW, RB, ARGMAX, ST>(p, grid, s);
    case 5: return launch_k<QT, 5, NW, RB, ARGMAX, ST>(p, grid, s);
    case 6: return launch_k<QT, 6, NW, RB, ARGMAX, ST>(p, grid, s);
    case 7: return launch_k<QT, 7, NW, RB, ARGMAX, ST>(p, grid, s);
    case 8: return launch_k<QT, 8, NW, RB, ARGMAX, ST>(p, grid, s);
    case 9: return launch_k<QT, 9, NW, RB, ARGMAX, ST>(p, grid, s);
    default: return launch_k<QT, 10, NW, RB, ARGMAX, ST>(p, grid, s);
  }
}

// Tile configurations (waves x row blocks of 16 rows, tokens):
//   cfg 1: 4 x 1 (64 rows), up to 160 tokens
//   cfg 2: 8 x 1 (128 rows), up to 160 tokens
//   cfg 3: 8 x 2 (256 rows), up to 80 tokens
//   cfg 4: 4 x 2 (128 rows), up to 80 tokens, two work-groups per CU
//   cfg 5: 4 x 1 (64 rows), up to 160 tokens, one activation stage, two
//          work-groups per CU
//   cfg 6: 4 x 1 (64 rows), up to 80 tokens, two work-groups per CU (the
//          cfg 1 kernel on at most five token blocks)
//   cfg 7: 12 x 1 (192 rows), up to 80 tokens (three waves per SIMD)
// The LM head (argmax) uses cfg 5: the same 64-row tiles as cfg 1, whose
// plain GEMM it outruns at the LM head's shapes (one activation stage, two
// work-groups per CU).
template <int QT>
static hipError_t launch_cfg(const GemmParams& p, int tb, int cfg, dim3 grid, bool argmax, hipStream_t s) {
  if (argmax) return launch_q<QT, 4, 1, true, 1>(p, tb, grid, s);
  if (cfg == 1 || cfg == 6) return launch_q<QT, 4, 1, false>(p, tb, grid, s);
  if (cfg == 2) return launch_q<QT, 8, 1, false>(p, tb, grid, s);
  if (cfg == 5) return launch_q<QT, 4, 1, false, 1>(p, tb, grid, s);
  if (cfg == 7) {
    switch (tb) {
      case 1: return launch_k<QT, 1, 12, 1, false>(p, grid, s);
      case 2: return launch_k<QT, 2, 12, 1, false>(p, grid, s);
      case 3: return launch_k<QT, 3, 12, 1, false>(p, grid, s);
      case 4: return launch_k<QT, 4, 12, 1, false>(p, grid, s);
      default: return launch_k<QT, 5, 12, 1, false>(p, grid, s);
    }
  }
  const bool c3 = (cfg == 3);
  switch (tb) {
    case 1: return c3 ? launch_k<QT, 1, 8, 2, false>(p, grid, s) : launch_k<QT, 1, 4, 2, false>(p, grid, s);
    case 2: return c3 ? launch_k<QT, 2, 8, 2, false>(p, grid, s) : launch_k<QT, 2, 4, 2, false>(p, grid, s);
    case 3: return c3 ? launch_k<QT, 3, 8, 2, false>(p, grid, s) : launch_k<QT, 3, 4, 2, false>(p, grid, s);
    case 4: return c3 ? launch_k<QT, 4, 8, 2, false>(p, grid, s) : launch_k<QT, 4, 4, 2, false>(p, grid, s);
    default: return c3 ? launch_k<QT, 5, 8, 2, false>(p, grid, s) : launch_k<QT, 5, 4, 2, false>(p, grid, s);
  }
}

// The SUMS form of each tile configuration, at its largest token tile.
template <int QT>
static hipError_t launch_sums_cfg(const GemmParams& p, int cfg, dim3 grid, hipStream_t s) {
  switch (cfg) {
    case 1: return launch_k<QT, 10, 4, 1, false, 2, true>(p, grid, s);
    case 2: return launch_k<QT, 10, 8, 1, false, 2, true>(p, grid, s);
    case 3: return launch_k<QT, 5, 8, 2, false, 2, true>(p, grid, s);
    case 4: return launch_k<QT, 5, 4, 2, false, 2, true>(p, grid, s);
    case 5: return launch_k<QT, 10, 4, 1, false, 1, true>(p, grid, s);
    case 6: return launch_k<QT, 5, 4, 1, false, 2, true>(p, grid, s);
    default: return launch_k<QT, 5, 12, 1, false, 2, true>(p, grid, s);
  }
}

hipError_t launch_qgemm_sums(int qtype, const GemmParams& p, int cfg, dim3 grid, hipStream_t s) {
  if (qtype == QT_Q4K) return launch_sums_cfg<QT_Q4K>(p, cfg, grid, s);
  return launch_sums_cfg<QT_Q6K>(p, cfg, grid, s);
}

// The grouped pairs that have a kernel: a Q4_K configuration-6 tile of 80
// tokens with a Q6_K tile of configuration 5 (160 tokens) or 6 (80 tokens);
// A and B in either order.
namespace {
using PairQ4c6 = Cfg4<QT_Q4K, 5, 2>;
using PairQ6c5 = Cfg4<QT_Q6K, 10, 1>;
using PairQ6c6 = Cfg4<QT_Q6K, 5, 2>;

int pair_kind(int qa, int cfg_a, int tb_a, int qb, int cfg_b, int tb_b) {
  if (qa != QT_Q4K || cfg_a != 6 || tb_a != 5 || qb != QT_Q6K) return 0;
  if (cfg_b == 5 && tb_b == 10) return 1;
  if (cfg_b == 6 && tb_b == 5) return 2;
  return 0;
}
}  // namespace

bool qgemm_pair_fits(int qtype_a, int cfg_a, int tb_a, int qtype_b, int cfg_b, int tb_b) {
  return pair_kind(qtype_a, cfg_a, tb_a, qtype_b, cfg_b, tb_b) != 0 ||
         pair_kind(qtype_b, cfg_b, tb_b, qtype_a, cfg_a, tb_a) != 0;
}

hipError_t launch_qgemm_pair(int qtype_a, const GemmParams& pa, int tb_a, int cfg_a, dim3 grid_a, int qtype_b,
                             const GemmParams& pb, int tb_b, int cfg_b, dim3 grid_b, hipStream_t s) {
  const bool swap = pair_kind(qtype_a, cfg_a, tb_a, qtype_b, cfg_b, tb_b) == 0;
  const int kind = swap ? pair_kind(qtype_b, cfg_b, tb_b, qtype_a, cfg_a, tb_a)
                        : pair_kind(qtype_a, cfg_a, tb_a, qtype_b, cfg_b, tb_b);
  if (kind == 0) return hipErrorInvalidValue;
  const GemmParams& p0 = swap ? pb : pa;
  const GemmParams& p1 = swap ? pa : pb;
  const dim3 g0 = swap ? grid_b : grid_a, g1 = swap ? grid_a : grid_b;
  PairGrid g{};
  g.n[0] = (int64_t)g0.x * g0.y * g0.z;
  g.n[1] = (int64_t)g1.x * g1.y * g1.z;
  g.gx[0] = g0.x;
  g.gy[0] = g0.y;
  g.gx[1] = g1.x;
  g.gy[1] = g1.y;
  g.groups[0] = (g.n[0] + 7) / 8;
  g.groups[1] = (g.n[1] + 7) / 8;
  const dim3 grid((unsigned)(8 * (g.groups[0] + g.groups[1])));
  if (kind == 1) hipLaunchKernelGGL((k_qgemm_pair<PairQ4c6, PairQ6c5>), grid, dim3(256), 0, s, p0, p1, g);
  else hipLaunchKernelGGL((k_qgemm_pair<PairQ4c6, PairQ6c6>), grid, dim3(256), 0, s, p0, p1, g);
  return hipGetLastError();
}

int qgemm_cfg_rows(int cfg) {
  return (cfg == 1 || cfg == 5 || cfg == 6) ? 64 : (cfg == 3 ? 256 : (cfg == 7 ? 192 : 128));
}
int qgemm_cfg_max_tb(int cfg) { return (cfg == 3 || cfg == 4 || cfg == 6 || cfg == 7) ? 5 : 10; }

hipError_t launch_qgemm(int qtype, const GemmParams& p, int tb, int cfg, dim3 grid, bool argmax, hipStream_t s) {
  if (qtype == QT_Q4K) return launch_cfg<QT_Q4K>(p, tb, cfg, grid, argmax, s);
  return launch_cfg<QT_Q6K>(p, tb, cfg, grid, argmax, s);
}

hipError_t launch_argmax_finalize(const uint64_t* keys, const float2* stats, int64_t n_tiles, int64_t M,
                                  int32_t* argmax, float* lse, float* p_max, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_finalize, dim3((unsigned)M), dim3(256), 0, s, keys, stats, n_tiles, M, argmax, lse,
                     p_max);
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
