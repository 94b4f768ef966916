// Device-side building blocks of the route kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace route {

constexpr int kHidden = 7168;   // K
constexpr int kLatent = 3584;   // N
constexpr int kExperts = 896;   // E
constexpr int kTopK = 16;
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// FP32 -> BF16, round to nearest even; NaN stays a quiet NaN with its sign.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// FP64 -> BF16 with a single nearest-even rounding. The FP64 value is first
// taken to FP32 with round-to-odd (sticky low bit), which keeps 16 more bits
// than BF16 in both the normal and the subnormal range, so the following FP32
// -> BF16 nearest-even step rounds exactly as a direct FP64 -> BF16 would.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
  if (d != d) return (uint16_t)((__double2hiint(d) >> 16 & 0x8000) | 0x7FC0);
  float f = (float)d;
  uint32_t u = __float_as_uint(f);
  double back = (double)f;
  if (back != d) {
    if (fabs(back) > fabs(d)) u -= 1u;   // step the magnitude back toward zero
    u |= 1u;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------- wave primitives --

// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int Ctrl, int RowMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // lanes without a source (or in masked rows) keep their own value
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, Ctrl, RowMask, 0xF, false);
}

// Maximum of an unsigned value over the 64 lanes, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kRowShr1, 0xF>(v));
  v = max(v, dpp_u32<kRowShr2, 0xF>(v));
  v = max(v, dpp_u32<kRowShr4, 0xF>(v));
  v = max(v, dpp_u32<kRowShr8, 0xF>(v));        // lane 15 of each row: row max
  v = max(v, dpp_u32<kRowBcast15, 0xA>(v));     // rows 1,3 take row 0,2's max
  v = max(v, dpp_u32<kRowBcast31, 0xC>(v));     // rows 2,3 take lane 31's max
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// --------------------------------------------------------------- top-16 --

// Unsigned key whose order is the logit order: -0.0 maps onto +0.0, NaN onto 0
// (below -inf, whose key is 0x007FFFFF).
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if ((b & 0x7FFFFFFFu) == 0u) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  uint64_t hi = a > b ? a : b;
  uint64_t lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// One wave selects the 16 largest of a row's 896 logits and writes ids and
// normalised sigmoid weights. Lane l owns experts l, l+64, ..., l+832 and keeps
// them as 64-bit keys (logit key << 32 | ~index), sorted descending with a
// Batcher odd-even merge network. Sixteen rounds then take the wave-wide
// largest head: a DPP max over the 32-bit logit keys, a ballot for the lanes
// that hold it, and (only on an exact logit tie) a second max over the index
// half to pick the lowest expert index. The winner pops its head.
// Coherent selects the load used for the logits: a device-scope atomic load
// when other workgroups of the same kernel wrote them (the fused epilogue).
template <bool Coherent = false>
__device__ __forceinline__ float load_logit(const float* p) {
  if constexpr (Coherent)
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

template <bool Coherent = false>
__device__ __forceinline__ void topk16_wave(const float* __restrict__ row, int32_t* __restrict__ ids,
                                            float* __restrict__ weights) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t c[16];
#pragma unroll
  for (int i = 0; i < 14; ++i) {
    const uint32_t idx = (uint32_t)(i * kWave + lane);
    c[i] = ((uint64_t)logit_key(load_logit<Coherent>(row + idx)) << 32) | (uint64_t)(~idx);
  }
  c[14] = 0;
  c[15] = 0;
  // Batcher odd-even merge sort, 16 inputs, descending.
#pragma unroll
  for (int p = 1; p < 16; p <<= 1) {
#pragma unroll
    for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
      for (int j = k % p; j + k < 16; j += 2 * k) {
#pragma unroll
        for (int i = 0; i < k; ++i) {
          if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) cas_desc(c[i + j], c[i + j + k]);
        }
      }
    }
  }
  uint32_t my_idx = 0;
#pragma unroll 1
  for (int slot = 0; slot < kTopK; ++slot) {
    const uint32_t hk = (uint32_t)(c[0] >> 32);
    const uint32_t m = wave_max_u32(hk);
    uint64_t tied = ballot(hk == m);
    uint32_t lo_best;
    if (__builtin_popcountll(tied) == 1) {
      const int w = __builtin_ctzll(tied);
      lo_best = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c[0], w);
    } else {
      lo_best = wave_max_u32(hk == m ? (uint32_t)c[0] : 0u);
    }
    const bool win = (hk == m) && ((uint32_t)c[0] == lo_best);
    if (lane == slot) my_idx = min(~lo_best, (uint32_t)(kExperts - 1));  // always a real entry
    if (win) {
#pragma unroll
      for (int i = 0; i < 13; ++i) c[i] = c[i + 1];
      c[13] = 0;
    }
  }
  // Weights: sigmoid in FP64, normalised over the 16 selected (fixed tree).
  double s = 0.0;
  if (lane < kTopK) {
    const double v = (double)load_logit<Coherent>(row + my_idx);
    s = 1.0 / (1.0 + exp(-v));
  }
  double tot = s;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 16);
  if (lane < kTopK) {
    ids[lane] = (int32_t)my_idx;
    weights[lane] = (float)(s / tot);
  }
}

}  // namespace route
