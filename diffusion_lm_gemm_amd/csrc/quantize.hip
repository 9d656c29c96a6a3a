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
// into the 292-byte record at `out` (written only if `store`; its d only if
// also `store_d`); returns d (0 if not `store`).
__device__ __forceinline__ float quantize_block(const float (&v)[4], uint8_t* out, int lane, bool store,
                                               bool store_d = true) {
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
    if (lane == 0 && store_d) *(float*)out = d;
  }
  return store ? d : 0.0f;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace

// Modes of the quantizer: the block values are the row of x itself (PLAIN,
// with an optional row gather for the LM head), or a producer fused in front
// of it:
//   RMSNORM: the codes of z = f32(x * g) (g the norm weight), each block's d
//            times the row's r = f32(1 / sqrt(mean(x^2) + eps)), the sum of
//            squares in f64: the blocks of RMSNorm(x) with the common factor r
//            moved into the block scales;
//   SWIGLU:  the row holds gate (values 0..K) and up (K..2K); the values are
//            f32(gate * up / (1 + exp(-gate))), evaluated in f64.
enum { Q_PLAIN = 0, Q_RMSNORM = 1, Q_SWIGLU = 2 };
constexpr int RMS_SBMAX = 64;  // blocks per row in RMSNORM mode (K <= 16384)

struct QuantArgs {
  const float* x;
  int64_t ldx;
  const int32_t* rows;  // PLAIN: gather rows[m] (or null)
  int64_t n_src;        // with rows: rows of x; an index outside [0, n_src) is clamped into it
  int64_t SB;           // blocks per output row
  uint8_t* y;
  float* dmax;          // per row, the largest |d| (or null)
  const float* g;       // RMSNORM: norm weight [K]
  float eps;            // RMSNORM
};

__device__ __forceinline__ void load4(const float* p, bool vec, float (&v)[4]) {
  if (vec) {
    const float4 t = *(const float4*)p;
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i];
  }
}

// QU = blocks per wave in flight: a block index past the row loads the row's
// last block again and stores nothing.
template <int QU, int MODE>
__global__ __launch_bounds__(64 * QW) void k_quantize_q8k(QuantArgs a) {
#pragma clang fp contract(off)
  __shared__ float s_wmax[QW];
  __shared__ double s_ss[QW];
  __shared__ float s_dz[MODE == Q_RMSNORM ? RMS_SBMAX : 1];
  __shared__ float s_r;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t m = blockIdx.x, SB = a.SB, K = SB * QK;
  int64_t src_row = m;
  if (MODE == Q_PLAIN && a.rows) {
    const int64_t i = (int64_t)a.rows[m];
    src_row = i < 0 ? 0 : (i >= a.n_src ? a.n_src - 1 : i);  // never a read outside x
  }
  const float* xrow = a.x + src_row * a.ldx;
  // every lane's 16 bytes are aligned exactly when the row start is
  const bool vec = ((((uintptr_t)xrow) & 15) == 0) && (MODE != Q_SWIGLU || (K & 3) == 0);
  uint8_t* yrow = a.y + m * SB * Q8K_BYTES;
  float wmax = 0.0f;
  double ss = 0.0;
  for (int64_t sb0 = wv; sb0 < SB; sb0 += QW * QU) {
    float v[QU][4];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t sb = sb0 + QW * u < SB ? sb0 + QW * u : SB - 1;
      load4(xrow + sb * QK + 4 * lane, vec, v[u]);
      if constexpr (MODE == Q_RMSNORM) {
        float gv[4];
        load4(a.g + sb * QK + 4 * lane, (((uintptr_t)a.g) & 15) == 0, gv);
        const bool live = sb0 + QW * u < SB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss += live ? (double)v[u][i] * (double)v[u][i] : 0.0;
          v[u][i] = v[u][i] * gv[i];
        }
      } else if constexpr (MODE == Q_SWIGLU) {
        float up[4];
        load4(xrow + K + sb * QK + 4 * lane, vec, up);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double gd = (double)v[u][i];
          v[u][i] = (float)(gd * (double)up[i] / (1.0 + exp(-gd)));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t sb = sb0 + QW * u;
      const float d = quantize_block(v[u], yrow + sb * Q8K_BYTES, lane, sb < SB, MODE != Q_RMSNORM);
      if constexpr (MODE == Q_RMSNORM) {
        if (lane == 0 && sb < SB) s_dz[sb] = d;
      } else {
        wmax = fmaxf(wmax, __builtin_fabsf(d));
      }
    }
  }
  if constexpr (MODE == Q_RMSNORM) {
    // the row's factor r, then each block's d = r * d_z (r > 0, so the
    // largest |d| is r times the largest |d_z| after rounding as well)
    ss = wave_sum_f64(ss);
    if (lane == 0) s_ss[wv] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
#pragma unroll
      for (int k = 0; k < QW; ++k) t += s_ss[k];
      s_r = (float)(1.0 / sqrt(t / (double)K + (double)a.eps));
    }
    __syncthreads();
    const float r = s_r;
    for (int64_t sb = threadIdx.x; sb < SB; sb += 64 * QW) {
      const float d = r * s_dz[sb];
      *(float*)(yrow + sb * Q8K_BYTES) = d;
      wmax = fmaxf(wmax, __builtin_fabsf(d));
    }
    if (a.dmax) {
      // every block's d is written by threads of wave 0 (SB <= 64)
      wmax = __builtin_bit_cast(float, wave_max_bits(__builtin_bit_cast(uint32_t, wmax)));
      if (threadIdx.x == 0) a.dmax[m] = wmax;
    }
  } else if (a.dmax) {
    if (lane == 0) s_wmax[wv] = wmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float r = s_wmax[0];
#pragma unroll
      for (int k = 1; k < QW; ++k) r = fmaxf(r, s_wmax[k]);
      a.dmax[m] = r;
    }
  }
}

template <int MODE>
static hipError_t launch_mode(const QuantArgs& a, int64_t M, hipStream_t s) {
  // enough blocks in flight per wave to cover rows of up to 64 blocks in one
  // round (K = 4096: one per wave; K = 12288: three)
  const int64_t per_wave = (a.SB + QW - 1) / QW;
  const dim3 grid((unsigned)M), block(64 * QW);
  if (per_wave <= 1)
    hipLaunchKernelGGL((k_quantize_q8k<1, MODE>), grid, block, 0, s, a);
  else if (per_wave == 2)
    hipLaunchKernelGGL((k_quantize_q8k<2, MODE>), grid, block, 0, s, a);
  else if (per_wave == 3)
    hipLaunchKernelGGL((k_quantize_q8k<3, MODE>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_quantize_q8k<4, MODE>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_q8k(const float* x, int64_t ldx, const int32_t* rows, int64_t n_src, int64_t M, int64_t SB,
                               uint8_t* y, float* dmax, hipStream_t s) {
  return launch_mode<Q_PLAIN>(QuantArgs{x, ldx, rows, n_src, SB, y, dmax, nullptr, 0.0f}, M, s);
}

bool rmsnorm_quantize_fits(int64_t SB) { return SB <= RMS_SBMAX; }

hipError_t launch_rmsnorm_quantize_q8k(const float* x, int64_t ldx, int64_t M, int64_t SB, const float* g, float eps,
                                       uint8_t* y, float* dmax, hipStream_t s) {
  return launch_mode<Q_RMSNORM>(QuantArgs{x, ldx, nullptr, 0, SB, y, dmax, g, eps}, M, s);
}

hipError_t launch_swiglu_quantize_q8k(const float* gu, int64_t ldgu, int64_t M, int64_t SB, uint8_t* y, float* dmax,
                                      hipStream_t s) {
  return launch_mode<Q_SWIGLU>(QuantArgs{gu, ldgu, nullptr, 0, SB, y, dmax, nullptr, 0.0f}, M, s);
}

}  // namespace dllm
