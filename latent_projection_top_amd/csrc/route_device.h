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
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

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
// (below -inf, whose key is 0x007FFFFF). Adding +0.0 turns -0.0 into +0.0 and
// leaves every other number as it is (FP32 subnormals are kept: the kernels
// run in IEEE denormal mode, and without fast-math flags the compiler keeps
// the add, since x + 0.0 is not x for x = -0.0); then a
// positive value gets its top bit set and a negative one has every bit
// inverted. No compare but the NaN test, so the 14 keys of a lane do not queue
// on the condition register.
__device__ __forceinline__ uint32_t logit_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  const uint32_t flip = (uint32_t)((int32_t)b >> 31) | 0x80000000u;
  return v != v ? 0u : (b ^ flip);
}

// Inverse of logit_key up to the sign of zero and the NaN payload, neither of
// which changes the sigmoid: key 0 is NaN.
__device__ __forceinline__ float key_logit(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  uint64_t hi = a > b ? a : b;
  uint64_t lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// Coherent selects the load used for the logits: a device-scope atomic load
// when other workgroups of the same kernel wrote them (the fused epilogue).
template <bool Coherent = false>
__device__ __forceinline__ float load_logit(const float* p) {
  if constexpr (Coherent)
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// 64-bit selection key of expert idx: logit key << 32 | ~idx. Keys are
// distinct and their order is (logit descending, index ascending).
template <bool Coherent>
__device__ __forceinline__ uint64_t select_key(const float* row, uint32_t idx) {
  return ((uint64_t)logit_key(load_logit<Coherent>(row + idx)) << 32) | (uint64_t)(~idx);
}

// Fallback selection (many keys at or above the threshold: the largest logits
// crowded into a few lanes, or large exact ties): lane-local Batcher
// odd-even merge sort of the keys (padded to 16), then sixteen rounds that
// take the wave-wide largest head (DPP max over the 32-bit logit key, a
// ballot for the lanes that hold it, a second max over the index half on an
// exact tie) and pop it. Lane s < 16 gets the s-th key.
template <int P>
__device__ __forceinline__ uint64_t select16_rounds(const uint64_t (&keys)[P]) {
  static_assert(P >= 1 && P <= 14, "keys per lane");
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = i < P ? keys[i] : 0ull;
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
  uint64_t mine = 0;
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
    if (lane == slot) mine = ((uint64_t)m << 32) | lo_best;
    if (win) {
#pragma unroll
      for (int i = 0; i < 15; ++i) c[i] = c[i + 1];
      c[15] = 0;
    }
  }
  return mine;
}

// LDS (uint64 slots) one wave of select16 needs: 64 candidates + 8 zero pads,
// 16 selected, and a slot that takes the stores of lanes with no candidate
// (one more keeps each wave's area a multiple of 16 bytes).
constexpr int kTopkScratch = 72 + kTopK + 2;
constexpr int kTopkDiscard = 72 + kTopK;
constexpr int kRankBatch = 24;   // candidates every lane reads in one batch

// Population count of a wave-wide ballot (two 32-bit counts, so that the
// compare that follows stays a scalar instruction).
__device__ __forceinline__ uint32_t mask_count(uint64_t m) {
  return (uint32_t)__builtin_popcount((uint32_t)m) + (uint32_t)__builtin_popcount((uint32_t)(m >> 32));
}
__device__ __forceinline__ uint32_t ballot_count(bool p) { return mask_count(ballot(p)); }

// The largest t with at least `need` lanes holding v >= t among the lanes
// where `in` is true, i.e. the need-th largest v of those lanes, built bit by
// bit from the top (ballots and scalar counts only; measured faster than two
// bits per step with three ballots). As soon as exactly `need` lanes are at
// or above the prefix, the answer is the smallest v among them, one wave
// minimum away: on rows of random logits that happens after about 15 of the
// 32 bits.
__device__ __forceinline__ uint32_t nth_largest_u32(uint32_t v, bool in, uint32_t need) {
  uint32_t t = 0;
  bool exact = false;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    const uint32_t n = ballot_count(in && v >= c);
    if (n >= need) {
      t = c;
      if (n == need) {
        exact = true;
        break;
      }
    }
  }
  return exact ? ~wave_max_u32(in && v >= t ? ~v : 0u) : t;
}

// One wave selects the 16 largest of a set of distinct 64-bit keys, P per
// lane (a zero key is padding: it is below every real key). At least 16
// lanes must hold a real key. Returns, in lane s < 16, the s-th largest key.
//   1. Threshold: t0 = the 16th largest of the 64 lanes' largest logit
//      halves, found with a bitwise search (32 ballots), over a zero index
//      half; only when several lanes share that largest logit half does a
//      second search narrow the index half among them. At least 16 keys are
//      >= t0, and the top 16 are among them.
//   2. The keys >= t0 (typically about 20) are compacted into LDS in ballot
//      order; each ranks itself against all of them, and rank r < 16 is the
//      r-th selected key.
//   3. More than 64 keys >= t0 take the sort-and-rounds fallback, which
//      selects the same keys.
// Every step is written so that its LDS accesses and ballots are independent
// and can be in flight together: one wave runs this alone, so latency, not
// throughput, sets its time.
// scratch: kTopkScratch uint64 slots of LDS owned by this wave. Waves are
// independent (no workgroup barrier inside).
template <int P>
__device__ __forceinline__ uint64_t select16(const uint64_t (&c)[P], uint64_t* scratch) {
  const int lane = threadIdx.x & (kWave - 1);
  // lane maximum of the logit halves
  uint32_t hm = (uint32_t)(c[0] >> 32);
#pragma unroll
  for (int i = 1; i < P; ++i) hm = max(hm, (uint32_t)(c[i] >> 32));

  // 1. th is the 16th largest lane maximum of the logit halves: 16 lanes hold
  //    a key whose logit half is >= th, and a key below th has at least 16
  //    keys above it, so t0 = th:0 bounds the top 16 from below. When several
  //    lane maxima share the logit half th, the index halves of those lanes'
  //    64-bit maxima narrow it (otherwise every key of logit half th would
  //    become a candidate, e.g. all 896 of a row of zeros).
  const uint32_t th = nth_largest_u32(hm, true, kTopK);
  const uint64_t eq = ballot(hm == th);
  uint64_t t0 = (uint64_t)th << 32;
  if (mask_count(eq) != 1u) {
    uint64_t m[P];
#pragma unroll
    for (int i = 0; i < P; ++i) m[i] = c[i];
#pragma unroll
    for (int w = 1; w < P; w *= 2)
#pragma unroll
      for (int i = 0; i + w < P; i += 2 * w) m[i] = m[i + w] > m[i] ? m[i + w] : m[i];
    const uint32_t need = kTopK - ballot_count(hm > th);
    t0 |= nth_largest_u32((uint32_t)m[0], hm == th, need);
  }

  // 2. compaction: every ballot first, then the scalar prefix counts, then
  //    the stores
  uint64_t* cand = scratch;
  uint64_t* sel = scratch + 72;
  uint64_t msk[P];
  uint32_t base[P];
  uint32_t n = 0;  // keys >= t0 (wave-uniform)
#pragma unroll
  for (int i = 0; i < P; ++i) msk[i] = ballot(c[i] >= t0);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    base[i] = n;
    n += mask_count(msk[i]);
  }
  if (n > (uint32_t)kWave) return select16_rounds<P>(c);
  // (a lane without a candidate stores to the discard slot: no branches)
#pragma unroll
  for (int i = 0; i < P; ++i)
    cand[c[i] >= t0 ? base[i] + lanes_below(msk[i]) : (uint32_t)kTopkDiscard] = c[i];
  // zero pads: up to the first batch, and up to a multiple of 8 beyond it
  if ((uint32_t)lane >= n && lane < kRankBatch) cand[lane] = 0ull;
  if (n > (uint32_t)kRankBatch && lane < 8) cand[n + lane] = 0ull;

  // 3. rank: the first 24 candidates in one batch of loads, the rest (rare)
  //    8 at a time
  const uint64_t mine = (uint32_t)lane < n ? cand[lane] : 0ull;
  uint64_t v[kRankBatch];
#pragma unroll
  for (int j = 0; j < kRankBatch; j += 2) {
    const u64x2 q = *reinterpret_cast<const u64x2*>(cand + j);
    v[j] = q[0];
    v[j + 1] = q[1];
  }
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < kRankBatch; ++j) r += v[j] > mine ? 1u : 0u;
  for (uint32_t j = kRankBatch; j < n; j += 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) r += cand[j + q] > mine ? 1u : 0u;
  }
  if ((uint32_t)lane < n && r < (uint32_t)kTopK) sel[r] = mine;
  return lane < kTopK ? sel[lane] : 0ull;
}

// Sum over lanes 0..15 of an FP64 value (0 in lanes 16..63), the same in every
// lane: an inclusive scan within the first 16-lane row (shifts by 1, 2, 4, 8;
// a lane without a source adds 0) leaves the total in lane 15, which is then
// broadcast. The order of the additions is fixed.
template <int Ctrl>
__device__ __forceinline__ double dpp_shr_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, Ctrl, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), Ctrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double sum16_f64(double v) {
  v += dpp_shr_f64<kRowShr1>(v);
  v += dpp_shr_f64<kRowShr2>(v);
  v += dpp_shr_f64<kRowShr4>(v);
  v += dpp_shr_f64<kRowShr8>(v);
  return __longlong_as_double((long long)readlane_u64((uint64_t)__double_as_longlong(v), 15));
}

// Lanes s < 16 hold the s-th selected key: write the ids (selection order)
// and the weights, sigmoid in FP64 of the selected logit (recovered from its
// key) normalised over the 16 in a fixed order, rounded once to FP32.
__device__ __forceinline__ void write_selection(uint64_t k, int32_t* __restrict__ ids,
                                                float* __restrict__ weights) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t my_idx = min(~(uint32_t)k, (uint32_t)(kExperts - 1));
  double s = 0.0;
  if (lane < kTopK) {
    const double v = (double)key_logit((uint32_t)(k >> 32));
    s = 1.0 / (1.0 + exp(-v));
  }
  const double tot = sum16_f64(s);
  if (lane < kTopK) {
    ids[lane] = (int32_t)my_idx;
    weights[lane] = (float)(s / tot);
  }
}

// One wave selects the 16 largest of a row's 896 logits and writes ids (in
// selection order) and normalised sigmoid weights. Lane l owns experts l,
// l + 64, ..., l + 832 as distinct 64-bit keys.
template <bool Coherent = false>
__device__ __forceinline__ void topk16_wave(const float* __restrict__ row, int32_t* __restrict__ ids,
                                            float* __restrict__ weights, uint64_t* scratch) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[14];
#pragma unroll
  for (int i = 0; i < 14; ++i) v[i] = load_logit<Coherent>(row + i * kWave + lane);
  uint64_t c[14];
#pragma unroll
  for (int i = 0; i < 14; ++i)
    c[i] = ((uint64_t)logit_key(v[i]) << 32) | (uint64_t)(~(uint32_t)(i * kWave + lane));
  write_selection(select16<14>(c, scratch), ids, weights);
}

}  // namespace route
