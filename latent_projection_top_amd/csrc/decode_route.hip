// Decode route (1..20 rows): latent down projection + FP32 router logits +
// standalone top-16 in one weight-streaming kernel.
//
// What is computed (page "Optionally gather the Kimi3 prefill latent instead of
// reducing it", voipmonitor/flare pull request 16, Description, numerics
// bullet): every latent value is one FP32-accumulated dot product over the
// full K = 7168, rounded to BF16 once. On one GPU there is no exchange: K is
// split only to spread the 77 MB of weights over all compute units, and the
// partials are combined in FP64 in a fixed order before the single rounding.
// The router logits are FP32 (page "Use two row blocks for eight-row Kimi
// paired gathers", NVIDIA/hyperflare-inference pull request 265); each row's
// experts are chosen by the standalone top-16 (page "Kimi K3.1 recipe: route
// 9..20 decode rows through the pushed pair gather and standalone top-16",
// voipmonitor/flare pull request 24, "What / why").
//
// Work split, described for [K][N] weights at 1..4 rows (4 latent x 16
// router K splits). Above 4 rows the [K][N] launch splits the router 8 ways
// (KnWideShape, 448 workgroups); packed weights split K 8 ways for both
// weights up to 4 rows and 4 (latent) / 8 (router) ways above (PackedShape,
// PackedWideShape); the 8-way router launches hold their latent stream back
// (latent_hold_ticks). A tensor-parallel rank's share uses the same units
// over its columns with more K splits. Every launch's workgroups are
// resident at once; here 672 workgroups of 4 waves:
//   workgroups 0..447, dispatched first: router units, expert tile (32
//       experts) x K chunk of 448 rows; each wave streams 112 rows (14,336
//       bytes) of the FP32 router weight and the unit stores one FP64 partial
//       per (row, expert); the last unit of a tile sums the 16 partials;
//   workgroups 448..671: latent units, column tile (64 columns) x K chunk of
//       1792 rows; each wave streams 448 rows (57,344 bytes) of the BF16 latent
//       weight; the last unit of a tile sums the 4 partials and rounds once.
// Router waves have a quarter of a latent wave's bytes (half with 8 router
// splits) and finish first; the workgroup that combines the last router tile
// then selects the top-16 of every row, four rows at a time (one per wave),
// while the latent weight is still streaming, and latent workgroups take any
// rows left when they finish.
// Nothing ever waits for another workgroup; every unit's arithmetic and
// combine order is fixed, so results do not depend on scheduling.
//
// Latent unit, per wave and 32-row step: each lane reads 8 rows x 4 columns
// (8-byte loads; 16 lanes cover one 128-byte row segment), transposes the 8x4
// BF16 block in registers with v_perm so that each of 4 registers holds 8
// consecutive-K values of one column, and issues 4 (8 for 17..20 rows)
// v_mfma_f32_16x16x32_bf16 with the hidden rows on the N side (padded to 16 or
// 32 inside the MFMA only). FP32 accumulation; the unit's 4 waves are summed in
// FP64; the last unit of a tile sums the 4 partials in FP64 and rounds once.
//
// Router unit, per wave and 16-row step: v_mfma_f64_16x16x4_f64 with the FP32
// weights and the BF16 hidden values widened exactly to FP64 (rows 16..19 as
// FP64 FMAs on the VALU), so the logits are accumulated in FP64 end to end and
// rounded to FP32 once.
#include "route.h"
#include "route_device.h"
#include "route_launch.h"

#include <mutex>

namespace route {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;              // 256
constexpr int kStepL = 32;                            // latent rows per MFMA step
constexpr int kLatTileN = 64;                         // latent columns per unit
constexpr int kStepR = 16;                            // router rows per step
constexpr int kRtTileE = 32;                          // experts per router unit
constexpr int kDecodeMaxRows = 20;
constexpr int kRowGroup = kWaves;                     // rows selected together, one per wave

// Output shape of one launch: the whole route (N = 3584 latent columns, E =
// 896 experts), or one tensor-parallel rank's share of it, whose weights are
// the rank's contiguous column slices: N = 448, E = 112 at 8 ranks; N = 224,
// E = 56 at 16 ranks (page "Optionally gather the Kimi3 prefill latent
// instead of reducing it", Description: 448 latent columns per rank; page "Use
// two row blocks for eight-row Kimi paired gathers": BF16 [8, 224] latent and
// FP32 [8, 56] router output per rank). A share has a few MB
// of weights, so it splits K further to spread them over the CUs; partial
// tiles at the end of a share are masked.
template <int N_, int E_, int SplitsL_, int SplitsR_>
struct DecodeShape {
  static constexpr int N = N_;                        // row stride of W, latent columns
  static constexpr int E = E_;                        // row stride of Wr, experts
  static constexpr bool kFull = N == kLatent && E == kExperts;
  // latent units: column tile x K split
  static constexpr int SplitsL = SplitsL_;
  static constexpr int KL = kHidden / SplitsL;        // rows per unit (1792 whole)
  static constexpr int KLWave = KL / kWaves;          // rows per wave (448)
  static constexpr int StepsL = KLWave / kStepL;      // MFMA steps per wave (14)
  static constexpr int LatTiles = (N + kLatTileN - 1) / kLatTileN;
  static constexpr int LatUnits = LatTiles * SplitsL;
  // router units: expert tile x K split
  static constexpr int SplitsR = SplitsR_;
  static constexpr int KR = kHidden / SplitsR;        // rows per unit (448 whole)
  static constexpr int KRWave = KR / kWaves;          // rows per wave (112)
  static constexpr int StepsR = KRWave / kStepR;      // MFMA steps per wave (7)
  static constexpr int RtTiles = (E + kRtTileE - 1) / kRtTileE;
  static constexpr int RtUnits = RtTiles * SplitsR;
  static constexpr int Grid = RtUnits + LatUnits;     // one workgroup per unit
  // Workspace counters (uint32). Every counter is shared by few workgroups:
  // atomics on one address from hundreds of workgroups serialise.
  static constexpr int CtrRtTile = LatTiles;          // router units stored per tile
  static constexpr int CtrPar = LatTiles + RtTiles;   // parity of the call (whole route)
  // two 8-byte-aligned pairs {router tiles combined, row groups claimed}, one
  // per call parity
  static constexpr int CtrPair = (CtrPar + 2) & ~1;
  static constexpr int Counters = CtrPair + 4;
  static_assert(KL * SplitsL == kHidden && KR * SplitsR == kHidden, "the splits cover K");
  static_assert(KLWave % kStepL == 0 && KRWave % kStepR == 0, "whole steps per wave");
  static_assert(N % 4 == 0 && E % 2 == 0, "a lane's loads stay inside a row");
};
using FullShape = DecodeShape<kLatent, kExperts, 4, 16>;
// With packed weights every unit's block is contiguous and any K split reads
// contiguous ranges, so the split is chosen by rows (graph over 8 weight
// copies, us per route, each with the latent hold and router prefetch below):
//   rows          1     2     4     8    12    16    17    20
//   8 x 8       17.5  17.5  18.0  18.8  19.5  20.2  21.7  21.8
//   4 x 8       18.0  18.0  18.0  18.5  19.2  19.7  21.0  21.2
//   4 x 16      18.7    -     -   20.0  20.9  20.9    -   22.9
// 8 x 8 gives every wave the same 28 KB to stream; 4 x 8 gives the latent
// waves twice the router waves' bytes. With [K][N] weights (each wave's loads
// are 128-byte row segments) 4 x 16 is faster up to 4 rows and 4 x 8 with the
// latent hold and router prefetch above (us per route, 1 / 8 / 12 / 16 / 20
// rows, 4 x 16: 18.1 / 20.4-20.8 / 21.3 / 22.0 / 24.0; 4 x 8: 18.4 / 19.6-19.7
// / 20.5-20.6 / 21.3-21.5 / 23.7-24.0; 4 x 8 without the hold 18.6 / 19.8 /
// 20.6 / 21.3 / 24.6).
using PackedShape = DecodeShape<kLatent, kExperts, 8, 8>;      // 1..4 rows
using PackedWideShape = DecodeShape<kLatent, kExperts, 4, 8>;  // 5..20 rows
using KnWideShape = DecodeShape<kLatent, kExperts, 4, 8>;      // [K][N] weights, 5..20 rows
constexpr int kNarrowMaxRows = 4;

// Latent units of a launch with 8 router splits hold their stream back
// after they start, 2.6 us up to 16 rows and 3.6 us at 17..20 rows (ticks of
// the 100 MHz realtime counter), so that the router's stream, which feeds the
// longer chain of dependent steps (tile combine, router completion, top-16),
// has the memory to itself first; the latent units, whose chain after the
// stream is shorter, still end in time. Measured (8 x 8, 1 / 4 / 8 rows):
// 17.2 / 18.1 / 19.0 us against 18.2 / 18.9 / 19.15 without it; holds of 2.0
// and 3.2 us were slower than 2.6. 4 x 8 at 17 / 20 rows: 26.2 / 25.5 us
// without a hold, 25.3 / 25.0 with 1.8 us, 22.7 / 22.6 with 2.6, 21.0 / 21.2
// with 3.6 and 21.4 / 21.9 with 4.5. With [K][N] weights (4 x 8) 2.6 us is
// also best up to 16 rows, and 17..20 rows take 4.2 us (17 / 20 rows
// 23.0-23.2 / 23.2 us against 23.4 / 23.5-23.8 with 3.6 and 23.7-24.2 /
// 23.8-24.1 with 3.0; 5.0 us 23.0-23.2 / 23.2-23.3). With 16
// router splits (the router stream already ends first) a hold did not help.
// A bounded wait on a clock, not on another workgroup.
template <int NT, class Sh, bool Packed>
constexpr uint64_t latent_hold_ticks() {
  return Sh::SplitsR != 8 ? 0 : NT == 1 ? 260 : Packed ? 360 : 420;
}

// Router steps of loads kept in flight per wave. With 8 router splits a
// router wave has 14 steps and, while the latent units hold, the memory to
// itself: all 14 in flight up to 16 rows (8 / 12 rows 0.3 us faster than 7),
// 10 at 17..20 rows (14 spill registers there). Otherwise up to 7 (all of a
// 16-split router wave's).
template <int NT, class Sh>
constexpr int router_depth() {
  const int d = Sh::SplitsR == 8 ? (NT == 1 ? 14 : 10) : 7;
  return Sh::StepsR < d ? Sh::StepsR : d;
}
// Share splits measured on MI355X (graph-replayed launches over 616 MB of
// distinct shares): with the tile combine's loads all in flight, fewer and
// longer K chunks won over 28 latent / 56 router splits by 1.5 to 3 us at 8
// ranks (7 / 28: 7.4 / 8.3 / 11.5 us at 1 / 8 / 20 rows; 14 / 28, 14 / 14,
// 7 / 14 and 28 / 28 were 0.4-1.9 us slower); the 16-rank share's four
// latent tiles take 28 splits (28 / 28: 7.1 / 7.8 / 11.0 us against 7.4 /
// 7.9 / 11.1 with 14 / 28).
using Tp8Shape = DecodeShape<448, 112, 7, 28>;
using Tp16Shape = DecodeShape<224, 56, 28, 28>;
constexpr int kDecodeCounters = FullShape::Counters;   // the largest counter set
constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
static_assert(Tp8Shape::Counters <= kDecodeCounters && Tp16Shape::Counters <= kDecodeCounters &&
                  PackedShape::Counters == kDecodeCounters && PackedWideShape::Counters == kDecodeCounters &&
                  KnWideShape::Counters == kDecodeCounters,
              "every shape's counters fit the workspace's counter area");
static_assert(FullShape::LatTiles == 56 && FullShape::RtTiles == 28 && FullShape::Grid == 672, "full shape");

// Rows a workgroup keeps in its LDS reduction buffer: the MFMA pads rows to 16
// or 32, but only real rows (at most 20) are stored.
template <int NT>
constexpr int rows_kept() { return NT == 1 ? 16 : kDecodeMaxRows; }

// Latent steps of loads kept in flight per wave (fewer at 17..20 rows, where
// the second set of hidden-row fragments and accumulators needs registers).
template <int NT>
constexpr int depth() { return NT == 1 ? 4 : 3; }

// Outputs per thread whose partials one tile combine loads together: enough
// for every output the thread has (the most rows of the variant times the
// tile width, over the workgroup's threads), within `budget` loaded values.
template <int NT, int TileW>
constexpr int combine_batch(int splits, int budget) {
  const int need = ((NT == 1 ? 16 : kDecodeMaxRows) * TileW + kThreads - 1) / kThreads;
  const int fit = budget / splits > 0 ? budget / splits : 1;
  return need < fit ? need : fit;
}

struct DecodeArgs {
  const uint16_t* __restrict__ x;
  const uint16_t* __restrict__ w;
  const float* __restrict__ wr;
  uint16_t* __restrict__ latent;
  float* __restrict__ logits;
  int32_t* __restrict__ ids;
  float* __restrict__ weights;
  float* __restrict__ lat_part;   // [SplitsL][rows_cap][N]
  double* __restrict__ rt_part;   // [SplitsR][rows_cap][E]
  uint32_t* __restrict__ counters;
  int rows;
  int rows_cap;
  int fuse_topk;
};

// Cross-workgroup handoff without device-wide cache maintenance. Each XCD has
// its own L2 and a device-scope fence would write back and invalidate the whole
// L2 for every workgroup. Instead, everything one workgroup hands to another
// (partials, counters) moves through device-scope relaxed atomic stores and
// loads, which the compiler emits with the sc1 bit so that they are coherent
// across XCDs; a store is complete once vmcnt drains.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's outstanding vector memory operations (stores
// included: GFX9 counts them in vmcnt) have completed.
__device__ __forceinline__ void drain_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Broadcast thread 0's value to the workgroup.
__device__ __forceinline__ int broadcast(int v, int* slot) {
  if (threadIdx.x == 0) *slot = v;
  __syncthreads();
  const int r = *slot;
  __syncthreads();
  return r;
}

// All threads' st_dev stores complete, then thread 0 adds 1 to `counter`;
// every thread gets the previous value.
__device__ __forceinline__ uint32_t publish(uint32_t* counter, int* slot) {
  drain_vmem();
  __syncthreads();
  int prev = 0;
  if (threadIdx.x == 0) prev = (int)add_dev(counter, 1u);
  return (uint32_t)broadcast(prev, slot);
}

// MFMA output column r only depends on hidden row r, and columns r >= rows are
// never stored, so padding lanes load a valid row (the last) without a branch:
// a branch here would drain the weight loads in flight at its join.
template <int NT>
__device__ __forceinline__ void hidden_rows(const DecodeArgs& a, int m, int (&xr)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) xr[nt] = min(16 * nt + m, a.rows - 1);
}

// Router rows 16..19 (17..20-row calls) on the FP64 VALU instead of a second
// 16-row MFMA block: the MFMA would pad 4 rows to 16, and FP64 MFMA and VALU
// have the same peak on this chip, so the VALU does the 4 rows at a quarter of
// the cost. Their hidden values for the unit's K chunk are staged in LDS.
constexpr int kTailRows = kDecodeMaxRows - 16;

// Returns true in the workgroup that combined the last router tile: every
// logit of every row is then stored.
template <int NT, class Sh, bool Packed>
__device__ bool router_unit(const DecodeArgs& a, const int u, char* smem, int* slot, uint32_t* pair) {
  constexpr bool kTail = NT == 2;                     // rows 16..19 on the VALU
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int m = lane & 15;
  constexpr int kRowsPad = rows_kept<NT>();
  int xr[1];
  hidden_rows<1>(a, m, xr);

  const int tile = u % Sh::RtTiles;
  const int split = u / Sh::RtTiles;
  const int e0 = tile * kRtTileE;
  const int k0 = split * Sh::KR + wave * Sh::KRWave;
  // lanes past the last expert of a share read a valid pair; never stored
  const int ecol = Sh::E % kRtTileE == 0 ? e0 + 2 * m : min(e0 + 2 * m, Sh::E - 2);
  // packed: a tile's K steps are consecutive 512-float blocks, and lane l's
  // two 16-byte pieces of a step sit at l and 64 + l (see pack_router_kernel)
  const float* wp = Packed ? a.wr + ((size_t)tile * (kHidden / kStepR) + k0 / kStepR) * (kStepR * kRtTileE) + 4 * lane
                           : a.wr + (size_t)(k0 + 4 * g) * Sh::E + ecol;

  // LDS after the reduction buffer: hidden rows 16..19 over the unit's K chunk
  uint16_t* xt = reinterpret_cast<uint16_t*>(smem + kWaves * kRowsPad * kRtTileE * 8);
  constexpr int kTailChunks = kTailRows * Sh::KR / 8;  // 16-byte pieces
  constexpr int kTailPer = (kTailChunks + kThreads - 1) / kThreads;
  u32x4 xtv[kTailPer];
#pragma unroll
  for (int q = 0; q < kTailPer; ++q) {
    const int t = threadIdx.x + q * kThreads;
    xtv[q] = u32x4{0u, 0u, 0u, 0u};
    if (kTail && t < kTailChunks) {
      const int i = t / (Sh::KR / 8);
      const int c = t % (Sh::KR / 8);
      xtv[q] = *(const u32x4*)(a.x + (size_t)min(16 + i, a.rows - 1) * kHidden + split * Sh::KR + 8 * c);
    }
  }

  f64x4 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
  double tacc[kTailRows][2];
#pragma unroll
  for (int i = 0; i < kTailRows; ++i) tacc[i][0] = tacc[i][1] = 0.0;
  constexpr int kDepthR = router_depth<NT, Sh>();
  f32x2 wv[kDepthR][4];
  u32x2 xv[kDepthR];
  auto issue = [&](int st) {
    if constexpr (Packed) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 v = __builtin_nontemporal_load((const f32x4*)(wp + st * (kStepR * kRtTileE) + h * 256));
        wv[st % kDepthR][2 * h] = f32x2{v[0], v[1]};
        wv[st % kDepthR][2 * h + 1] = f32x2{v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wv[st % kDepthR][j] =
            __builtin_nontemporal_load((const f32x2*)(wp + (size_t)(st * kStepR + j) * Sh::E));
    }
    xv[st % kDepthR] = *(const u32x2*)(a.x + (size_t)xr[0] * kHidden + k0 + 4 * g + st * kStepR);
  };
  // router_depth() steps of loads in flight: all 7 of a 4 x 16 router wave's
  // (measured: 0.3 us faster at 8 rows and 0.5 us at 20 rows than 4 steps
  // ahead, at the same register count), 14 or 10 of an 8 x 8 wave's
#pragma unroll
  for (int st = 0; st < kDepthR; ++st) issue(st);
  __builtin_amdgcn_sched_barrier(0);  // keep the prefetch where it is issued
  if (kTail) {
#pragma unroll
    for (int q = 0; q < kTailPer; ++q) {
      const int t = threadIdx.x + q * kThreads;
      if (t < kTailChunks) {
        const int i = t / (Sh::KR / 8);
        const int c = t % (Sh::KR / 8);
        *(u32x4*)(xt + i * Sh::KR + 8 * c) = xtv[q];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int st = 0; st < Sh::StepsR; ++st) {
    const int q = st % kDepthR;
    // lane (g, m) at step j: A[m][g] = Wr[k][e0 + 2m + c], B[g][m] = x[row m][k],
    // k = k0 + 16*st + 4*g + j
    u32x2 xtl[kTailRows];
    if (kTail) {
#pragma unroll
      for (int i = 0; i < kTailRows; ++i)
        xtl[i] = *(const u32x2*)(xt + i * Sh::KR + wave * Sh::KRWave + st * kStepR + 4 * g);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double w0 = (double)wv[q][j][0];
      const double w1 = (double)wv[q][j][1];
      const double xd = (double)((j & 1) ? bf16_hi(xv[q][j >> 1]) : bf16_lo(xv[q][j >> 1]));
      acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(w0, xd, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w1, xd, acc[1], 0, 0, 0);
      if (kTail) {
#pragma unroll
        for (int i = 0; i < kTailRows; ++i) {
          const double xi = (double)((j & 1) ? bf16_hi(xtl[i][j >> 1]) : bf16_lo(xtl[i][j >> 1]));
          tacc[i][0] = fma(w0, xi, tacc[i][0]);
          tacc[i][1] = fma(w1, xi, tacc[i][1]);
        }
      }
    }
    if (st + kDepthR < Sh::StepsR) issue(st + kDepthR);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kTail) {
    // lane (g, m) summed K rows 4g..4g+3 of each step: add the four g groups
#pragma unroll
    for (int i = 0; i < kTailRows; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        tacc[i][c] += __shfl_xor(tacc[i][c], 16);
        tacc[i][c] += __shfl_xor(tacc[i][c], 32);
      }
  }

  double* red = reinterpret_cast<double*>(smem);
  // The FP64 MFMA keeps D[4*t + g][m] in slot t of lane (g, m): lane (g, m)
  // holds row m, local experts 2*(4*t + g) + c = 8*t + 2*g + c.
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      red[(wave * kRowsPad + m) * kRtTileE + 8 * t + 2 * g + c] = acc[c][t];
  if (kTail && g == 0) {
#pragma unroll
    for (int i = 0; i < kTailRows; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) red[(wave * kRowsPad + 16 + i) * kRtTileE + 2 * m + c] = tacc[i][c];
  }
  __syncthreads();
  const int outs = a.rows * kRtTileE;
  for (int i = threadIdx.x; i < outs; i += kThreads) {
    const int r = i / kRtTileE;
    const int e = i % kRtTileE;
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[(w * kRowsPad + r) * kRtTileE + e];
    if (Sh::E % kRtTileE == 0 || e0 + e < Sh::E)
      st_dev(&a.rt_part[((size_t)split * a.rows_cap + r) * Sh::E + e0 + e], s);
  }
  if (publish(&a.counters[Sh::CtrRtTile + tile], slot) != (uint32_t)(Sh::SplitsR - 1)) return false;
  // Last unit of this tile: each logit is the sum of its partials in split
  // order. Every coherent load is a round trip to memory, so a thread loads
  // the partials of all its outputs (up to 48 values) before adding any.
  constexpr int kJB = combine_batch<NT, kRtTileE>(Sh::SplitsR, 48);
  for (int i0 = threadIdx.x; i0 < outs; i0 += kJB * kThreads) {
    double p[kJB][Sh::SplitsR];
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      // past the last output or expert: load a valid partial, store nothing
      const int i = min(i0 + j * kThreads, outs - 1);
      const int r = i / kRtTileE;
      const int e = min(e0 + i % kRtTileE, Sh::E - 1);
#pragma unroll
      for (int q = 0; q < Sh::SplitsR; ++q)
        p[j][q] = ld_dev(&a.rt_part[((size_t)q * a.rows_cap + r) * Sh::E + e]);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first add
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      const int i = i0 + j * kThreads;
      const int r = i / kRtTileE;
      const int e = e0 + i % kRtTileE;
      if (i >= outs || (Sh::E % kRtTileE != 0 && e >= Sh::E)) continue;
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < Sh::SplitsR; ++q) s += p[j][q];
      st_dev(&a.logits[(size_t)r * Sh::E + e], (float)s);
    }
  }
  if (threadIdx.x == 0) st_dev(&a.counters[Sh::CtrRtTile + tile], 0u);
  return publish(&pair[0], slot) == (uint32_t)(Sh::RtTiles - 1);
}

template <int NT, class Sh, bool Packed>
__device__ bool latent_unit(const DecodeArgs& a, const int u, char* smem, int* slot) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int m = lane & 15;
  constexpr int kRowsPad = rows_kept<NT>();
  int xr[NT];
  hidden_rows<NT>(a, m, xr);

  const int tile = u % Sh::LatTiles;
  const int split = u / Sh::LatTiles;
  const int n0 = tile * kLatTileN;
  const int k0 = split * Sh::KL + wave * Sh::KLWave;
  // lanes past the last column of a share read a valid quad; never stored
  const int ncol = Sh::N % kLatTileN == 0 ? n0 + 4 * m : min(n0 + 4 * m, Sh::N - 4);
  // packed: a tile's K steps are consecutive 2048-value blocks, and lane l's
  // piece for MFMA c sits at 64 c + l (see pack_latent_kernel)
  const uint16_t* wp = Packed ? a.w + ((size_t)tile * (kHidden / kStepL) + k0 / kStepL) * (kStepL * kLatTileN) + 8 * lane
                              : a.w + (size_t)(k0 + 8 * g) * Sh::N + ncol;

  f32x4 acc[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (latent_hold_ticks<NT, Sh, Packed>() > 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < latent_hold_ticks<NT, Sh, Packed>())
      __builtin_amdgcn_s_sleep(2);
  }
  constexpr int kDepth = depth<NT>() < Sh::StepsL ? depth<NT>() : Sh::StepsL;
  u32x2 wv[kDepth][8];
  u32x4 wq[kDepth][4];
  u32x4 xv[kDepth][NT];
  auto issue = [&](int st) {
    if constexpr (Packed) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        wq[st % kDepth][c] =
            __builtin_nontemporal_load((const u32x4*)(wp + st * (kStepL * kLatTileN) + c * 512));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        wv[st % kDepth][j] =
            __builtin_nontemporal_load((const u32x2*)(wp + (size_t)(st * kStepL + j) * Sh::N));
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      xv[st % kDepth][nt] = *(const u32x4*)(a.x + (size_t)xr[nt] * kHidden + k0 + 8 * g + st * kStepL);
  };
#pragma unroll
  for (int st = 0; st < kDepth; ++st) issue(st);
  __builtin_amdgcn_sched_barrier(0);  // keep the prefetch where it is issued
#pragma unroll
  for (int st = 0; st < Sh::StepsL; ++st) {
    const int q = st % kDepth;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 av;
      if constexpr (Packed) {
        av = wq[q][c];
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          av[p] = __builtin_amdgcn_perm(wv[q][2 * p + 1][c >> 1], wv[q][2 * p][c >> 1], sel);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv[q][nt]), acc[nt][c], 0, 0, 0);
    }
    if (st + kDepth < Sh::StepsL) issue(st + kDepth);
    __builtin_amdgcn_sched_barrier(0);
  }

  float* red = reinterpret_cast<float*>(smem);
  // lane (g, m) holds row 16*nt + m, local columns 16*g + 4*t + c
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (16 * nt + m < kRowsPad)
          red[(wave * kRowsPad + 16 * nt + m) * kLatTileN + 16 * g + 4 * t + c] = acc[nt][c][t];
  __syncthreads();
  const int outs = a.rows * kLatTileN;
  for (int i = threadIdx.x; i < outs; i += kThreads) {
    const int r = i / kLatTileN;
    const int col = i % kLatTileN;
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += (double)red[(w * kRowsPad + r) * kLatTileN + col];
    if (Sh::N % kLatTileN == 0 || n0 + col < Sh::N)
      st_dev(&a.lat_part[((size_t)split * a.rows_cap + r) * Sh::N + n0 + col], (float)s);
  }
  if (publish(&a.counters[tile], slot) != (uint32_t)(Sh::SplitsL - 1)) return false;
  // Last unit of this tile: the partials in split order, summed in FP64 and
  // rounded once; a thread loads the partials of all its outputs (up to 32
  // values) before adding any.
  constexpr int kJB = combine_batch<NT, kLatTileN>(Sh::SplitsL, 32);
  for (int i0 = threadIdx.x; i0 < outs; i0 += kJB * kThreads) {
    float p[kJB][Sh::SplitsL];
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      // past the last output or column: load a valid partial, store nothing
      const int i = min(i0 + j * kThreads, outs - 1);
      const int r = i / kLatTileN;
      const int n = min(n0 + i % kLatTileN, Sh::N - 1);
#pragma unroll
      for (int q = 0; q < Sh::SplitsL; ++q)
        p[j][q] = ld_dev(&a.lat_part[((size_t)q * a.rows_cap + r) * Sh::N + n]);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first add
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      const int i = i0 + j * kThreads;
      const int r = i / kLatTileN;
      const int n = n0 + i % kLatTileN;
      if (i >= outs || (Sh::N % kLatTileN != 0 && n >= Sh::N)) continue;
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < Sh::SplitsL; ++q) s += (double)p[j][q];
      a.latent[(size_t)r * Sh::N + n] = f64_to_bf16_rne(s);
    }
  }
  if (threadIdx.x == 0) st_dev(&a.counters[tile], 0u);
  return true;
}

// Row group: rows r0..r0+3 (those below `rows`). Every logit is stored; for
// the fused call wave w selects the top-16 of row r0 + w, reading the logits
// with coherent loads (other workgroups of this launch wrote them).
__device__ void row_group(const DecodeArgs& a, const int r0, char* smem) {
  uint64_t* scratch = reinterpret_cast<uint64_t*>(smem);
  const int nr = min(kRowGroup, a.rows - r0);
  const int w = threadIdx.x >> 6;
  if (w < nr)
    topk16_wave<true>(a.logits + (size_t)(r0 + w) * kExperts, a.ids + (size_t)(r0 + w) * kTopK,
                      a.weights + (size_t)(r0 + w) * kTopK, scratch + w * kTopkScratch);
  __syncthreads();
}

// A latent workgroup's first claim of a row group. Group 0 (rows 0..3)
// belongs to the workgroup that completed the router, which starts on it
// without a claim; pair[1] hands out the later groups. The latent workgroup
// first reads the pair in one coherent load and claims only if the router is
// complete and a group is left. Returns the group's first row, or -1. Thread
// 0 holds `pair`.
template <class Sh>
__device__ __forceinline__ int first_claim(const DecodeArgs& a, uint32_t* pair, int* slot) {
  int r = -1;
  if (threadIdx.x == 0) {
    const uint64_t v = ld_dev(reinterpret_cast<const uint64_t*>(pair));
    if ((uint32_t)v == (uint32_t)Sh::RtTiles && kRowGroup + (uint32_t)(v >> 32) < (uint32_t)a.rows) {
      const uint32_t c = kRowGroup + add_dev(&pair[1], (uint32_t)kRowGroup);
      if (c < (uint32_t)a.rows) r = (int)c;
    }
  }
  return broadcast(r, slot);
}

// Workgroup b < Sh::RtUnits (448 for the whole route) runs router unit b, the
// others latent unit b - Sh::RtUnits.
//
// Row phase (the fused top-16 of the whole route). Row groups are taken by
// the workgroup that combines the last router tile, until none is left, and
// by any workgroup that combines a latent tile after the logits are complete.
// Nobody waits and nobody counts the participants out: the two counters of
// the phase live in one of two pairs chosen by the call's parity, which
// thread 0 of every workgroup reads at its start. The workgroup that
// completed the router, after its last group, clears the other pair (last
// used by the previous call, which has ended) and flips the parity for the
// next call. Every router unit reads the parity before its tile can be
// combined, so every increment of this call's router counter lands in this
// call's pair; a latent workgroup that read the flipped parity would only
// find a cleared pair and take no row.
template <int NT, class Sh, bool Packed>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void decode_route_kernel(DecodeArgs a) {
  static_assert(!Packed || Sh::kFull, "packed weights cover the whole route");
  constexpr int kLatBytes = kWaves * rows_kept<NT>() * kLatTileN * 4;
  constexpr int kRtBytes = kWaves * rows_kept<NT>() * kRtTileE * 8 +
                           (NT == 2 ? kTailRows * Sh::KR * 2 : 0);   // + staged hidden rows
  constexpr int kRowBytes = kRowGroup * kTopkScratch * 8;
  constexpr int kB0 = kLatBytes > kRtBytes ? kLatBytes : kRtBytes;
  constexpr int kBytes = kB0 > kRowBytes ? kB0 : kRowBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];
  __shared__ int slot;

  const int b = blockIdx.x;
  uint32_t par = 0;
  if (Sh::kFull && threadIdx.x == 0) par = ld_dev(&a.counters[Sh::CtrPar]) & 1u;
  uint32_t* pair = &a.counters[Sh::CtrPair + 2 * par];
  bool router_done = false;
  if (b < Sh::RtUnits) {
    router_done = router_unit<NT, Sh, Packed>(a, b, smem, &slot, pair);
    if (!router_done) return;
  } else if (!latent_unit<NT, Sh, Packed>(a, b - Sh::RtUnits, smem, &slot)) {
    return;
  }
  if constexpr (!Sh::kFull) {
    // A share has no row phase (its experts are a fraction of the route's, so
    // there is nothing to select): the workgroup that combined the last router
    // tile clears the router counter, and the call ends.
    if (router_done && threadIdx.x == 0) st_dev(&pair[0], 0u);
    return;
  }
  int r = !a.fuse_topk ? -1 : router_done ? 0 : first_claim<Sh>(a, pair, &slot);
  while (r >= 0) {
    // Groups are handed out in order: none is left after the one that ends
    // at or past the last row. Otherwise thread 0 claims the next group once
    // this one is selected, not before: a latent workgroup that finishes its
    // combine meanwhile then takes it and the two groups run side by side
    // (measured: 8 / 9 / 12 rows 0.3 / 0.45 / 0.8 us faster than claiming as
    // soon as the group's logit loads are issued, 20 rows no slower).
    const bool more = r + kRowGroup < a.rows;
    row_group(a, r, smem);
    uint32_t c = ~0u;
    if (more && threadIdx.x == 0) c = kRowGroup + add_dev(&pair[1], (uint32_t)kRowGroup);
    r = broadcast(threadIdx.x == 0 && c < (uint32_t)a.rows ? (int)c : -1, &slot);
  }
  if (router_done && threadIdx.x == 0) {
    uint32_t* other = &a.counters[Sh::CtrPair + 2 * (par ^ 1u)];
    st_dev(&other[0], 0u);
    st_dev(&other[1], 0u);
    st_dev(&a.counters[Sh::CtrPar], par ^ 1u);
  }
}

// Sh2: a second shape sharing the workspace (the whole route's packed
// launches share the [K][N] launch's counters and partial areas); each
// partial area fits the larger of the two.
template <class Sh, class Sh2 = Sh>
static size_t ws_bytes(int rows_cap, size_t* off_lat, size_t* off_rt, size_t* off_logits, size_t* off_cand) {
  constexpr int kSL = Sh::SplitsL > Sh2::SplitsL ? Sh::SplitsL : Sh2::SplitsL;
  constexpr int kSR = Sh::SplitsR > Sh2::SplitsR ? Sh::SplitsR : Sh2::SplitsR;
  static_assert(Sh::N == Sh2::N && Sh::E == Sh2::E, "shapes sharing a workspace");
  size_t off = align256(sizeof(uint32_t) * kDecodeCounters);
  *off_lat = off;
  off = align256(off + sizeof(float) * kSL * (size_t)rows_cap * Sh::N);
  *off_rt = off;
  off = align256(off + sizeof(double) * kSR * (size_t)rows_cap * Sh::E);
  *off_logits = off;
  off = align256(off + sizeof(float) * (size_t)rows_cap * Sh::E);
  *off_cand = off;
  off = align256(off + sizeof(uint64_t) * (size_t)rows_cap * kTopkMaxShards * kTopK);
  return off;
}

bool decode_shape_valid(int latent, int experts) {
  return (latent == FullShape::N && experts == FullShape::E) ||
         (latent == Tp8Shape::N && experts == Tp8Shape::E) ||
         (latent == Tp16Shape::N && experts == Tp16Shape::E);
}

size_t decode_workspace_bytes(int rows_cap, int latent, int experts, size_t* off_lat, size_t* off_rt,
                              size_t* off_logits, size_t* off_cand) {
  if (latent == Tp8Shape::N && experts == Tp8Shape::E)
    return ws_bytes<Tp8Shape>(rows_cap, off_lat, off_rt, off_logits, off_cand);
  if (latent == Tp16Shape::N && experts == Tp16Shape::E)
    return ws_bytes<Tp16Shape>(rows_cap, off_lat, off_rt, off_logits, off_cand);
  static_assert(PackedWideShape::SplitsL <= PackedShape::SplitsL &&
                    PackedWideShape::SplitsR <= FullShape::SplitsR &&
                    KnWideShape::SplitsL <= PackedShape::SplitsL && KnWideShape::SplitsR <= FullShape::SplitsR,
                "the 4 x 8 launches fit the partial areas of the other two");
  return ws_bytes<FullShape, PackedShape>(rows_cap, off_lat, off_rt, off_logits, off_cand);
}

template <class Sh, bool Packed = false>
static hipError_t launch_shape(const DecodeArgs& a, int rows, hipStream_t stream) {
  if (rows <= 16)
    return launch_kernel(decode_route_kernel<1, Sh, Packed>, dim3(Sh::Grid), dim3(kThreads), stream, a);
  return launch_kernel(decode_route_kernel<2, Sh, Packed>, dim3(Sh::Grid), dim3(kThreads), stream, a);
}

hipError_t launch_decode_route(const uint16_t* x, const uint16_t* w_latent, const float* w_router,
                               uint16_t* latent, float* logits, int32_t* ids, float* weights,
                               const DecodeWorkspace& ws, int rows, int rows_cap, int n_latent,
                               int n_experts, bool fuse_topk, bool packed, hipStream_t stream) {
  if (rows < 1 || rows > kDecodeMaxRows || rows > rows_cap) return hipErrorInvalidValue;
  if (!decode_shape_valid(n_latent, n_experts)) return hipErrorInvalidValue;
  const bool full = n_latent == FullShape::N;
  if ((fuse_topk || packed) && !full) return hipErrorInvalidValue;
  DecodeArgs a;
  a.x = x;
  a.w = w_latent;
  a.wr = w_router;
  a.latent = latent;
  a.logits = logits;
  a.ids = ids;
  a.weights = weights;
  a.lat_part = ws.lat_part;
  a.rt_part = ws.rt_part;
  a.counters = ws.counters;
  a.rows = rows;
  a.rows_cap = rows_cap;
  a.fuse_topk = fuse_topk ? 1 : 0;
  if (full && packed && rows <= kNarrowMaxRows) return launch_shape<PackedShape, true>(a, rows, stream);
  if (full && packed) return launch_shape<PackedWideShape, true>(a, rows, stream);
  if (full && rows <= kNarrowMaxRows) return launch_shape<FullShape>(a, rows, stream);
  if (full) return launch_shape<KnWideShape>(a, rows, stream);
  if (n_latent == Tp8Shape::N) return launch_shape<Tp8Shape>(a, rows, stream);
  return launch_shape<Tp16Shape>(a, rows, stream);
}

// ----------------------------------------------------- static device scratch --
//
// Scratch of the allocation-free entry point (route_fused_packed_noalloc),
// for callers that cannot allocate device memory: this code object's device
// global, one copy per GPU, held until the process ends. Layout for the
// packed launches at up to 20 decode rows: the counter area, the latent
// partials [8 splits][20][3584] FP32, the router partials [8 splits][20][896]
// FP64, then a logits buffer [20][896] FP32. Every call on a GPU shares its
// copy; the decode kernels leave the counters in the state the next call
// expects, so it is cleared once, when the first plan for the device is
// prepared. The kernels receive its address, never the array's name (in
// host code the name is a host-side stand-in, not a device address).
constexpr size_t kStaticOffLat = align256(sizeof(uint32_t) * kDecodeCounters);
constexpr size_t kStaticOffRt =
    kStaticOffLat + align256(sizeof(float) * PackedShape::SplitsL * kDecodeMaxRows * kLatent);
constexpr size_t kStaticOffLogits =
    kStaticOffRt + align256(sizeof(double) * PackedShape::SplitsR * kDecodeMaxRows * kExperts);
constexpr size_t kStaticBytes = kStaticOffLogits + align256(sizeof(float) * kDecodeMaxRows * kExperts);
static_assert(PackedWideShape::SplitsL <= PackedShape::SplitsL &&
                  PackedWideShape::SplitsR <= PackedShape::SplitsR,
              "both packed launches fit the static partial areas");

static_assert(kStaticBytes == ROUTE_STATIC_SCRATCH_BYTES, "the size the header states");

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch_init(int device) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_static_ptr[device] != nullptr) return hipSuccess;
  int prev = -1;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return e;
  if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  // cleared once (the decode counters must start at zero), before any call
  // on this device can use it
  if (e == hipSuccess) e = hipMemset(p, 0, kStaticBytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) g_static_ptr[device] = p;
  if (prev != device) {
    const hipError_t r = hipSetDevice(prev);
    if (e == hipSuccess) e = r;
  }
  return e;
}

void* static_scratch(int device, size_t* bytes) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  *bytes = kStaticBytes;
  return device >= 0 && device < kMaxDevices ? g_static_ptr[device] : nullptr;
}

DecodeWorkspace static_decode_workspace(void* base, float** logits) {
  char* b = static_cast<char*>(base);
  DecodeWorkspace d;
  d.counters = reinterpret_cast<uint32_t*>(b);
  d.lat_part = reinterpret_cast<float*>(b + kStaticOffLat);
  d.rt_part = reinterpret_cast<double*>(b + kStaticOffRt);
  *logits = reinterpret_cast<float*>(b + kStaticOffLogits);
  return d;
}

size_t static_free_offset() { return kStaticOffLat; }

// ------------------------------------------------------------ weight packing --
//
// The packed decode weights hold the same values as W [7168][3584] BF16 and
// Wr [7168][896] FP32, reordered once (at weight load) into the order in which
// the whole-route kernel's lanes consume them, so that every unit streams one
// contiguous block and every load instruction covers 1 KB with one 16-byte
// piece per lane. Each tile's data is in K order, so that a unit of any K
// split reads one contiguous range. The packed kernel splits K its own ways
// (PackedShape, PackedWideShape) where the [K][N] kernel splits the latent 4
// and the router 16 ways, so the latent's last bit may differ from
// route_fused's (both are one full-K dot rounded once, within the same
// bounds); its logits are FP64 sums rounded once, as there.
//
// Latent: tile t (64 columns), K step s (32 rows), MFMA c, lane (g, m) =
// (l / 16, l mod 16): 8 BF16 values W[32 s + 8 g + i][64 t + 4 m + c],
// i = 0..7, at value offset (((t*224 + s)*4 + c)*64 + l)*8.
// Router: tile t (32 experts), K step s (16 rows), half h, lane (g, m):
// {Wr[k][e], Wr[k][e+1], Wr[k+1][e], Wr[k+1][e+1]} with k = 16 s + 4 g + 2 h
// and e = 32 t + 2 m, at float offset (((t*448 + s)*2 + h)*64 + l)*4.
constexpr int kPackLatPieces = kHidden * kLatent / 8;    // 16-byte pieces
constexpr int kPackRtPieces = kHidden * kExperts / 4;

__global__ __launch_bounds__(256) void pack_latent_kernel(const uint16_t* __restrict__ w,
                                                          uint16_t* __restrict__ out) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= kPackLatPieces) return;
  const int l = p % 64;
  const int c = (p / 64) % 4;
  const int s = (p / 256) % (kHidden / kStepL);
  const int tile = p / (256 * (kHidden / kStepL));
  const int k = kStepL * s + 8 * (l >> 4);
  const int n = tile * kLatTileN + 4 * (l & 15) + c;
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (uint32_t)w[(size_t)(k + 2 * i) * kLatent + n] |
           ((uint32_t)w[(size_t)(k + 2 * i + 1) * kLatent + n] << 16);
  *(u32x4*)(out + (size_t)p * 8) = v;
}

__global__ __launch_bounds__(256) void pack_router_kernel(const float* __restrict__ wr,
                                                          float* __restrict__ out) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= kPackRtPieces) return;
  const int l = p % 64;
  const int h = (p / 64) % 2;
  const int s = (p / 128) % (kHidden / kStepR);
  const int tile = p / (128 * (kHidden / kStepR));
  const int k = kStepR * s + 4 * (l >> 4) + 2 * h;
  const int e = tile * kRtTileE + 2 * (l & 15);
  const f32x2 r0 = *(const f32x2*)(wr + (size_t)k * kExperts + e);
  const f32x2 r1 = *(const f32x2*)(wr + (size_t)(k + 1) * kExperts + e);
  *(f32x4*)(out + (size_t)p * 4) = f32x4{r0[0], r0[1], r1[0], r1[1]};
}

static_assert(kPackLatPieces == FullShape::LatTiles * (kHidden / kStepL) * 4 * 64,
              "the latent pieces cover every tile, K step, MFMA and lane");
static_assert(kPackRtPieces == FullShape::RtTiles * (kHidden / kStepR) * 2 * 64,
              "the router pieces cover every tile, K step, half and lane");

size_t decode_packed_latent_bytes() { return (size_t)kHidden * kLatent * 2; }
size_t decode_packed_bytes() { return decode_packed_latent_bytes() + (size_t)kHidden * kExperts * 4; }

hipError_t launch_pack_decode_weights(const uint16_t* w_latent, const float* w_router, void* packed,
                                      hipStream_t stream) {
  uint16_t* lat = static_cast<uint16_t*>(packed);
  float* rt = reinterpret_cast<float*>(static_cast<char*>(packed) + decode_packed_latent_bytes());
  const hipError_t e = launch_kernel(pack_latent_kernel, dim3((kPackLatPieces + 255) / 256), dim3(256),
                                     stream, w_latent, lat);
  if (e != hipSuccess) return e;
  return launch_kernel(pack_router_kernel, dim3((kPackRtPieces + 255) / 256), dim3(256), stream, w_router, rt);
}

}  // namespace route
