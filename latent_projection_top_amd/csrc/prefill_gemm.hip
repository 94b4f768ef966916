// Prefill route (up to 3072 rows): latent down projection and router logits as
// two MFMA GEMMs over the hidden rows.
//
// Page "Optionally gather the Kimi3 prefill latent instead of reducing it"
// (voipmonitor/flare pull request 16), Description: in a prefill MoE layer
// every latent value is computed from the full hidden row (K = 7168) as one
// FP32-accumulated dot product and rounded to BF16 once; the GEMM shape is
// M = prefill rows, K = 7168 (the page's per-rank N is 448; one GPU computes
// all N = 3584 columns).
//
// Latent: C[M][3584] = x[M][7168] * W[7168][3584] on v_mfma_f32_16x16x32_bf16.
// A running FP32 MFMA accumulator loses accuracy with the length of its chain
// (each step rounds into a sum that keeps growing), so the accumulators start
// from zero every 256 K values and are added into a second FP32 sum; the
// result is rounded to BF16 once, nearest-even.
//
// Router: logits[M][896] = x * Wr with Wr in FP32. A small pass splits each
// FP32 weight exactly into three BF16 parts (w = hi + mid + lo: each step
// takes the top 8 significant bits of what is left; the remainder after two
// steps has at most 8 significant bits) and stores them as a BF16 matrix
// [7168][14 expert groups][3 parts][64 experts]. x is BF16, so every product
// x * part is exact in FP32 and the contraction is a BF16 GEMM with 2688
// columns. The hi products run in one FP32 chain, the mid and lo products in
// another (they are 2^-8 smaller and more), both restarted every 256 K values
// and folded into FP64 sums that are rounded once to FP32.
//
// Tiling for gfx950 (256 CUs): block tile 192 rows x 224 columns (latent) or
// 192 x 192 (router: 64 experts x 3 parts), so 3072 rows give 256 latent
// blocks, one per CU; chunks of few row tiles also split K over more blocks
// (prefill_splits), and some chunk sizes take 128-row tiles instead
// (prefill_gemm_plan). Eight waves, 4 x 2, each 48 (or 32) rows x (112 | 96)
// columns with its accumulators in VGPRs: two waves per SIMD keep the matrix
// core busy where one wave holding everything in AGPRs reaches only about 55%
// of its rate. K step 64, three LDS stages (156 KB at most). Operands go from
// global memory straight to LDS (global_load_lds_dwordx4: 64 lanes x 16
// bytes land contiguously), so no staging registers are spent on them:
//   A stage [192 rows][64 k]: 128-byte rows, the 16-byte piece c of row r
//     stored at position c ^ ((r >> 1) & 7), so the 16 rows one MFMA lane
//     group reads hit 16 different bank groups;
//   B stage [cols/32 blocks][64 k][32 cols], W keeps its [K][N] order: the
//     MFMA wants 8 consecutive K of one column per lane, which
//     ds_read_tr16_b64 delivers from row-major data (lane L of a 16-lane
//     group gets element L % 4 of the 8-byte chunks that lanes L / 4 + 4 j
//     address, j = 0..3). The two 32-byte halves of a 64-byte row are swapped
//     when (k >> 3) is odd, so the two lane groups of one read phase use
//     different banks.
//
// Packed weights (BT = true): the weights stored K-contiguous instead, W as
// [3584][7168] and the router's three BF16 parts as [2688][7168] (the parts
// split once, when the weights are packed, in the same column order). The B
// stage is then laid out like the A stage, [cols][64 k] with the same piece
// swizzle, and read with ds_read_b128 like A: twice the bytes per LDS read
// instruction of the transposing read. Every lane receives the same operand
// values in the same order as with the [K][N] weights, so the results are
// bitwise the same.
#include <type_traits>

#include "route_device.h"
#include "route_launch.h"

namespace route {

constexpr int kGBM = 192;             // rows of a block tile (or 128, below)
constexpr int kGBK = 64;
constexpr int kGStages = 3;
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGKT = kHidden / kGBK;   // 112 K stages
constexpr int kGFoldStages = 4;        // accumulators restart every 4 x 64 = 256 K
constexpr int kPrefillMaxRows = 3072;
constexpr int kRouterCols = 3 * kExperts;  // 2688: [14 groups][3 parts][64]

static_assert(kGKT % kGFoldStages == 0, "fold period");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

template <bool Router, int BMr>
struct GemmShape {
  static constexpr int BM = BMr;                     // block rows: 192, or 128
  static constexpr int BN = Router ? 192 : 224;      // block columns
  static constexpr int NT = Router ? 6 : 7;          // 16-column MFMA tiles per wave
  static constexpr int MT = BM / 64;                 // 16-row MFMA tiles per wave (4 row slices)
  static constexpr int NB = BN / 32;                 // 32-column B blocks per stage
  static constexpr int N = Router ? kRouterCols : kLatent;
  static constexpr int A_BYTES = BM * kGBK * 2;      // 24576 or 16384
  static constexpr int B_BYTES = NB * kGBK * 64;     // NB x 4096
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024;     // 1 KB loads per stage (block)
  static constexpr int B_LOADS = B_BYTES / 1024;
  static constexpr int LOADS = A_LOADS + B_LOADS;    // dealt round-robin over the waves
  static constexpr int PER_WAVE = (LOADS + kGWaves - 1) / kGWaves;
  static_assert(N % BN == 0, "column tiles");
  static_assert(A_LOADS % kGWaves == 0, "A loads come first and split evenly");
  static_assert(BM == 192 || BM == 128, "block rows");
  static_assert(kGStages * STAGE <= 160 * 1024, "LDS");
};

// Column (within the block tile) of the wave's n-tile j.
template <bool Router>
__device__ __forceinline__ constexpr int tile_col(int wn, int j) {
  return Router ? 64 * (j >> 1) + 32 * wn + 16 * (j & 1) : 112 * wn + 16 * j;
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  // s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt low
  // bits [3:0], high bits [15:14]; expcnt [6:4]; lgkmcnt [11:8])
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most `pending` of this wave's global -> LDS loads are in
// flight; a wave owns PER_WAVE or PER_WAVE - 1 loads of every stage.
template <int PerWave>
__device__ __forceinline__ void vm_wait_stages(bool full_wave, int stages_pending) {
  if (stages_pending == 2) {
    if (full_wave) vm_wait<2 * PerWave>(); else vm_wait<2 * (PerWave - 1)>();
  } else if (stages_pending == 1) {
    if (full_wave) vm_wait<PerWave>(); else vm_wait<PerWave - 1>();
  } else {
    vm_wait<0>();
  }
}

// One 16-byte-per-lane global -> LDS load: lane l's 16 bytes from
// base + voff land at LDS address lds + 16 l. Written as inline assembly so
// that the compiler does not add a wait for every outstanding load before
// each LDS read (it cannot tell the stages apart); the kernel waits with
// explicit vmcnt counts instead. M0 carries the LDS address.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "{m0}"(lds)
      : "memory");
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}

__device__ __forceinline__ s16x4 lds_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
}

__device__ __forceinline__ bool f32_nonfinite(float v) {
  return (__float_as_uint(v) & 0x7F800000u) == 0x7F800000u;
}

// Router logits the GEMM returned as an infinity or a NaN, recomputed exactly
// by the workgroup that computed them (or, for a K-split launch, that
// combined them).
//
// The GEMM multiplies the hidden row by three BF16 parts of each FP32 weight.
// The parts can differ in sign or be zero, so an infinite hidden value gives
// inf - inf or inf * 0 (NaN) where the single product x * w is an infinity;
// and an FP32 chain can overflow where the full float64 dot stays finite. A
// finite hidden row with no overflow never produces a non-finite logit, and
// an infinite or NaN hidden value makes every logit of its row non-finite.
// So every logit of the block's tile that came out non-finite is recomputed
// as a plain FP64 dot of the hidden row with the FP32 weight, rebuilt exactly
// as hi + mid + lo from the parts (each sum exact in FP64): waves 0..3 take
// one K quarter each for the tile's 64 experts, the four quarters are added
// in a fixed order and rounded once to FP32; finite logits keep the GEMM's
// value. mask[b] bit j: row bm0 + 64 b + j holds a non-finite logit of the
// tile. red: 256 doubles of LDS.
template <bool BT, int NW>
__device__ void router_recompute(const uint16_t* __restrict__ x, const uint16_t* __restrict__ parts,
                                 float* __restrict__ logits, int bm0, int group, const uint64_t (&mask)[NW],
                                 double* red) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int e = group * 64 + lane;
  const int kb = (wave & 3) * (kHidden / 4);
#pragma unroll 1
  for (int b = 0; b < NW; ++b) {
    uint64_t todo = mask[b];
    while (todo != 0) {
      const int r = bm0 + 64 * b + __builtin_ctzll(todo);
      todo &= todo - 1;
      if (wave < 4) {
        const uint16_t* xr = x + (size_t)r * kHidden;
        double s = 0.0;
        if constexpr (BT) {
          // part p of expert e: row group * 192 + 64 p + lane of [2688][7168]
          const uint16_t* ph = parts + (size_t)(group * 192 + lane) * kHidden;
          for (int k = kb; k < kb + kHidden / 4; k += 8) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + k);
            const u32x4 hv = *reinterpret_cast<const u32x4*>(ph + k);
            const u32x4 mv = *reinterpret_cast<const u32x4*>(ph + (size_t)64 * kHidden + k);
            const u32x4 lv = *reinterpret_cast<const u32x4*>(ph + (size_t)128 * kHidden + k);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int h = i >> 1;
              auto part = [&](uint32_t pair) { return (double)((i & 1) ? bf16_hi(pair) : bf16_lo(pair)); };
              const double w = part(hv[h]) + part(mv[h]) + part(lv[h]);
              s = fma(part(xv[h]), w, s);
            }
          }
        } else {
          // part p of expert e at [k][group * 192 + 64 p + lane] of [7168][2688]
          const uint16_t* pk = parts + group * 192 + lane;
#pragma unroll 8
          for (int k = kb; k < kb + kHidden / 4; ++k) {
            const uint16_t* q = pk + (size_t)k * kRouterCols;
            const double w = (double)__uint_as_float((uint32_t)q[0] << 16) +
                             (double)__uint_as_float((uint32_t)q[64] << 16) +
                             (double)__uint_as_float((uint32_t)q[128] << 16);
            s = fma((double)__uint_as_float((uint32_t)xr[k] << 16), w, s);
          }
        }
        red[(wave & 3) * 64 + lane] = s;
      }
      __syncthreads();
      if (wave == 0) {
        float* dst = logits + (size_t)r * kExperts + e;
        if (f32_nonfinite(*dst)) *dst = (float)(((red[lane] + red[64 + lane]) + red[128 + lane]) + red[192 + lane]);
      }
      __syncthreads();
    }
  }
}

template <bool Router, bool BT, int BM>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                         void* __restrict__ out, int rows, int mtiles, int nsplit, void* __restrict__ part) {
  using S = GemmShape<Router, BM>;
  __shared__ __attribute__((aligned(1024))) char smem[kGStages * S::STAGE];
  // router: rows of the tile with a non-finite logit (bit j of word b: row
  // bm0 + 64 b + j)
  __shared__ uint64_t bad_rows[Router ? BM / 64 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int m = lane & 15;
  const int wm = wave >> 1;  // row slice (16 MT rows)
  const int wn = wave & 1;   // column half

  // Tile order. The hardware deals blocks round-robin over the 8 XCDs, so
  // block b is first renumbered (b % 8) * (total / 8) + b / 8 (when that
  // divides evenly), giving each XCD a contiguous range; the range is then
  // walked in groups of 8 row tiles, column by column, so that one XCD's L2
  // holds about 8 A tiles and 4 B tiles at a time.
  // With nsplit > 1 (few row tiles) the blocks of K split q are the q-th run
  // of `total` blocks, each over K stages [q nkt, (q + 1) nkt), and write
  // their FP32 (latent) or FP64 (router) sums to `part` for a combine pass.
  const int ntiles = S::N / S::BN;
  const int total = mtiles * ntiles;
  const int split = blockIdx.x / total;
  const int bid = blockIdx.x - split * total;
  const int nkt = kGKT / nsplit;
  const int kt0 = split * nkt;
  const int kend = kt0 + nkt;
  int lin = bid;
  if ((total & 7) == 0) lin = (bid & 7) * (total >> 3) + (bid >> 3);
  const int grp = lin / (8 * ntiles);
  const int first = grp * 8;
  const int gm = min(mtiles - first, 8);
  const int loc = lin - grp * 8 * ntiles;
  const int bm0 = (first + loc % gm) * BM;
  const int bn0 = (loc / gm) * S::BN;

  // ---- global -> LDS loads: load c of a stage (wave c % 8) -----------------
  //   c < A_LOADS: A rows 8 c .. 8 c + 7;  else B block (c - A_LOADS) / 4,
  //   k rows 16 ((c - A_LOADS) % 4) .. + 15 ([K][N] weights), or B columns
  //   8 (c - A_LOADS) .. + 7 (K-contiguous weights, laid out like A).
  const bool full_wave = wave + kGWaves * (S::PER_WAVE - 1) < S::LOADS;
  // K-contiguous B: load i of a wave reads columns 64 (i - A_LOADS / 8) past
  // those of its first B load, with the same piece swizzle, so one offset
  // serves all of them and the column step goes on the scalar base
  constexpr int kAW = S::A_LOADS / kGWaves;             // A loads per wave
  constexpr size_t kBtStep = (size_t)kGWaves * 8 * kHidden * 2;
  uint32_t off[BT ? kAW + 1 : S::PER_WAVE];
#pragma unroll
  for (int i = 0; i < (BT ? kAW + 1 : S::PER_WAVE); ++i) {
    const int c = wave + kGWaves * i;
    if (c < S::A_LOADS) {
      const int r = 8 * c + (lane >> 3);
      const int piece = (lane & 7) ^ ((r >> 1) & 7);
      const int row = min(bm0 + r, rows - 1);
      off[i] = (uint32_t)(row * kHidden + 8 * piece) * 2u;
    } else if constexpr (BT) {
      const int ib = min(c, S::LOADS - 1) - S::A_LOADS;
      const int r = 8 * ib + (lane >> 3);
      const int piece = (lane & 7) ^ ((r >> 1) & 7);
      off[i] = (uint32_t)((bn0 + r) * kHidden + 8 * piece) * 2u;
    } else {
      const int ib = min(c, S::LOADS - 1) - S::A_LOADS;
      const int k = 16 * (ib & 3) + (lane >> 2);
      const int q = (lane & 3) ^ (((k >> 3) & 1) << 1);
      off[i] = (uint32_t)(k * S::N + bn0 + 32 * (ib >> 2) + 8 * q) * 2u;
    }
  }
  const char* a_src = reinterpret_cast<const char*>(x);
  const char* b_src = reinterpret_cast<const char*>(w);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;

  // `full`: this wave owns PER_WAVE loads of every stage (else PER_WAVE - 1);
  // the pipeline below is instantiated for both, so no stage tests it
  auto issue_one = [&](int kt, int i, bool full) {
    const uint32_t st = lds0 + (kt % kGStages) * S::STAGE;
    const char* ab = a_src + (size_t)kt * (kGBK * 2);
    const char* bb = b_src + (BT ? (size_t)kt * (kGBK * 2) : (size_t)kt * ((size_t)kGBK * S::N * 2));
    const int c = wave + kGWaves * i;
    if (i < kAW)
      dma16(ab, off[i], st + c * 1024);
    else if (i < S::PER_WAVE - 1 || full) {
      if constexpr (BT)
        dma16(bb + (size_t)(i - kAW) * kBtStep, off[kAW], st + c * 1024);
      else
        dma16(bb, off[i], st + c * 1024);
    }
  };
  auto issue = [&](int kt, bool full) {
#pragma unroll
    for (int i = 0; i < S::PER_WAVE; ++i) issue_one(kt, i, full);
  };

  // ---- LDS -> register operand addresses ----------------------------------
  // A, tile i, K half s: row 16 MT wm + 16 i + m, piece 4 s + g (the swizzle
  // term (row >> 1) & 7 equals (m >> 1) & 7 because 16 MT wm + 16 i is a
  // multiple of 16).
  uint32_t a_rd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    a_rd[s] = (uint32_t)((16 * S::MT * wm + m) * 128 + (((4 * s + g) ^ ((m >> 1) & 7)) * 16));
  // B, 16-column half h of a 32-column block, K rows 8 g + m / 4 (+ 32 s + 4 e),
  // columns 16 h + 4 (m % 4) .. + 3.
  uint32_t b_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    b_rd[h] = (uint32_t)(S::A_BYTES + (8 * g + (m >> 2)) * 64 +
                         ((2 * (h ^ (g & 1)) + ((m & 3) >> 1)) * 16) + (m & 1) * 8);

  struct Ops {
    bf16x8 a[S::MT];
    bf16x8 b[S::NT];
  };
  auto read_a = [&](uint32_t st, int s, int i) { return lds_b128(st + a_rd[s] + 2048 * i); };
  // K-contiguous B, column c of the block, K half s: like A, row c (a multiple
  // of 16 plus m), piece 4 s + g
  // (the wave's column offset goes into the base, so that every tile's
  // offset is a constant the read instruction carries)
  uint32_t bt_rd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    bt_rd[s] = (uint32_t)(S::A_BYTES + (tile_col<Router>(wn, 0) + m) * 128 +
                          (((4 * s + g) ^ ((m >> 1) & 7)) * 16));
  auto read_b = [&](uint32_t st, int s, int j) -> bf16x8 {
    if constexpr (BT) {
      // tile_col(wn, j) = tile_col(wn, 0) + tile_col(0, j)
      return lds_b128(st + bt_rd[s] + 128 * tile_col<Router>(0, j));
    } else {
      const int col = tile_col<Router>(wn, j);
      const uint32_t base = st + b_rd[(col >> 4) & 1] + (col >> 5) * 4096 + 32 * s * 64;
      const s16x4 lo = lds_tr16(base);
      const s16x4 hi = lds_tr16(base + 4 * 64);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto stage_lds = [&](int kt) { return lds0 + (kt % kGStages) * S::STAGE; };

  // latent: one chain per tile; router: chains 0, 1 take the hi parts of the
  // two 16-expert tiles, chains 2, 3 their mid and lo parts
  f32x4 chain[S::MT][Router ? 4 : S::NT];
  f32x4 sum32[Router ? 1 : S::MT][Router ? 1 : S::NT];
  double sum64[Router ? S::MT : 1][Router ? 2 : 1][4];
#pragma unroll
  for (int i = 0; i < S::MT; ++i) {
    if constexpr (Router) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) sum64[i][j][t] = 0.0;
    } else {
#pragma unroll
      for (int j = 0; j < S::NT; ++j) sum32[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // One K half (32) of MFMAs, row by row. Each operand register is refilled
  // with the next K half's value as soon as its last MFMA has been issued
  // (a[i] after row i, b[j] in the last row), so the next half's operands
  // arrive while this half's MFMAs run, without a second register set.
  auto step = [&](Ops& o, bool restart, bool reload, uint32_t st_n, int s_n, int dma_kt, bool dma, bool full) {
#pragma unroll
    for (int i = 0; i < S::MT; ++i) {
#pragma unroll
      for (int j = 0; j < S::NT; ++j) {
        {
          // spread this wave's loads of stage dma_kt over the MFMAs: load d
          // goes out after MFMA kEvery * d + 1
          constexpr int kEvery = (S::MT * S::NT) / S::PER_WAVE;
          const int p = i * S::NT + j;
          if (dma && p % kEvery == 1 && p / kEvery < S::PER_WAVE) issue_one(dma_kt, p / kEvery, full);
        }
        if constexpr (Router) {
          const int c = j < 2 ? j : 2 + (j & 1);
          const bool z = restart && j < 4;  // first MFMA of each chain in the period
          chain[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[j], z ? zero4 : chain[i][c],
                                                               0, 0, 0);
        } else {
          chain[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[j],
                                                               restart ? zero4 : chain[i][j], 0, 0, 0);
        }
        if (reload && i == S::MT - 1) o.b[j] = read_b(st_n, s_n, j);
      }
      if (reload) o.a[i] = read_a(st_n, s_n, i);
    }
  };

  // Pipeline (three LDS stages, loads two stages ahead). The first K half of
  // stage kt runs while the second half's operands are read; then every wave
  // has read all of stage kt, waits for its own loads of stage kt + 1 and
  // meets the others at the barrier: past it, stage kt + 1 is complete in
  // LDS and stage kt's buffer takes the loads of stage kt + 3, while the
  // second half runs and reads the first half of stage kt + 1.
  // The pipeline is instantiated for full and short waves (a wave-uniform
  // choice made once), so that no stage branches on it.
  auto pipeline = [&](auto full_tag) {
    constexpr bool kFull = decltype(full_tag)::value;
    issue(kt0, kFull);
    issue(kt0 + 1, kFull);
    issue(kt0 + 2, kFull);
    if (Router && tid < BM / 64) bad_rows[tid] = 0;
    vm_wait_stages<S::PER_WAVE>(kFull, 2);
    __syncthreads();
    Ops o;
#pragma unroll
    for (int i = 0; i < S::MT; ++i) o.a[i] = read_a(stage_lds(kt0), 0, i);
#pragma unroll
    for (int j = 0; j < S::NT; ++j) o.b[j] = read_b(stage_lds(kt0), 0, j);

    // One fold period (kGFoldStages stages). Every period but the last has the
    // loads of the next two stages in flight at each wait and issues the loads
    // of stage kt + 3; the last period (Tail) drains them. With the tail
    // peeled, the steady-state stages carry no run-time conditions.
    auto period = [&](int kp, auto tail) {
      constexpr bool kTail = decltype(tail)::value;
#pragma unroll
      for (int u = 0; u < kGFoldStages; ++u) {
        const int kt = kp + u;
        step(o, u == 0, true, stage_lds(kt), 1, -1, false, kFull);
        lgkm_wait0();
        // (tail: kend - kp == kGFoldStages, so kt + 2 < kend is u < 2)
        vm_wait_stages<S::PER_WAVE>(kFull, !kTail || u < kGFoldStages - 2 ? 1 : 0);
        __syncthreads();
        // (after the last stage this reads a stale buffer; the values go unused)
        // Stage kt + 3's loads: spread over the second half's MFMAs, so that
        // the matrix core restarts right after the barrier (measured: latent
        // + router 239.9 against 245.8 us; packed latent GEMM 135.5 against
        // 141.7 us; [K][N] latent GEMM 130.3-131.0 against 143.1-146.1 us).
        const bool more = !kTail || u < kGFoldStages - 3;   // kt + 3 < kend
        step(o, false, true, stage_lds(kt + 1), 0, kt + 3, more, kFull);
      }
      // fold the restarted chains into the long sums
#pragma unroll
      for (int i = 0; i < S::MT; ++i) {
        if constexpr (Router) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              sum64[i][j][t] += (double)chain[i][j][t] + (double)chain[i][j + 2][t];
        } else {
#pragma unroll
          for (int j = 0; j < S::NT; ++j) sum32[i][j] += chain[i][j];
        }
      }
    };
#pragma unroll 1
    for (int kp = kt0; kp < kend - kGFoldStages; kp += kGFoldStages) period(kp, std::false_type{});
    period(kend - kGFoldStages, std::true_type{});
  };
  if (full_wave)
    pipeline(std::true_type{});
  else
    pipeline(std::false_type{});

  // lane (g, m) of tile (i, j) holds row 16 i + 4 g + t, column 16 j + m
  if (part != nullptr) {
    // split partials [nsplit][rows][N]: latent FP32, router FP64
#pragma unroll
    for (int i = 0; i < S::MT; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = bm0 + 16 * S::MT * wm + 16 * i + 4 * g + t;
        if (row >= rows) continue;
        if constexpr (Router) {
          const int e0 = (bn0 / 192) * 64 + 32 * wn + m;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            static_cast<double*>(part)[((size_t)split * rows + row) * kExperts + e0 + 16 * j] = sum64[i][j][t];
        } else {
#pragma unroll
          for (int j = 0; j < S::NT; ++j)
            static_cast<float*>(part)[((size_t)split * rows + row) * kLatent + bn0 + tile_col<false>(wn, j) + m] =
                sum32[i][j][t];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < S::MT; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = bm0 + 16 * S::MT * wm + 16 * i + 4 * g + t;
      if (row >= rows) continue;
      if constexpr (Router) {
        // expert group bn0 / 192, experts 32 wn + 16 j + m of its 64
        const int e0 = (bn0 / 192) * 64 + 32 * wn + m;
        bool bad = false;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float v = (float)sum64[i][j][t];
          static_cast<float*>(out)[(size_t)row * kExperts + e0 + 16 * j] = v;
          bad |= f32_nonfinite(v);
        }
        if (bad) {
          const int lr = row - bm0;
          atomicOr((unsigned long long*)&bad_rows[lr >> 6], 1ull << (lr & 63));
        }
      } else {
#pragma unroll
        for (int j = 0; j < S::NT; ++j) {
          const int col = bn0 + tile_col<false>(wn, j) + m;
          static_cast<uint16_t*>(out)[(size_t)row * kLatent + col] = f32_to_bf16_rne(sum32[i][j][t]);
        }
      }
    }
  }
  if constexpr (Router) {
    __syncthreads();
    uint64_t mask[BM / 64];
    uint64_t any = 0;
#pragma unroll
    for (int b = 0; b < BM / 64; ++b) any |= (mask[b] = bad_rows[b]);
    // (every stage's reads are done: the LDS stages are free)
    if (any != 0)
      router_recompute<BT, BM / 64>(x, w, static_cast<float*>(out), bm0, bn0 / 192, mask,
                                    reinterpret_cast<double*>(smem));
  }
}

// K splits for chunks of few row tiles. A GEMM block streams its whole
// weight tile (224 or 192 columns x 7168 K) through one CU, so with few row
// tiles the GEMMs use a fraction of the 256 CUs and take about as long as a
// full 3072-row chunk (measured 203-215 us per packed chunk for 64 to 2048
// rows unsplit). Splitting K fills the chip; the cost is the partials' round
// trip through HBM and a combine pass. The split of each GEMM by row tiles
// comes from a model of one block's full-K time and the partials' traffic,
// over splits whose K stages are whole fold periods (112 / S a multiple of
// 4), checked by measurement: packed chunks of 64 / 192 / 384 / 768 / 1024 /
// 1536 / 1728 rows take 40 / 52 / 64 / 88 / 129 / 144 / 187 us against 204 /
// 209 / 209 / 211 / 211 / 214 / 214 unsplit (A/B, one box; 2048 and 3072
// rows are not split and unchanged). Every output is still one sum over all
// of K rounded once: the combine adds the splits' FP32 (latent) or FP64
// (router) sums in split order in FP64. The split changes the order of the
// FP32 additions, so a row's last bit may depend on the chunk's row count.
static int prefill_splits(int mtiles, bool router) {
  if (mtiles <= 1) return 14;
  if (mtiles == 2) return 7;
  if (mtiles <= 4) return 4;
  if (mtiles <= 8 || (router && mtiles == 9)) return 2;
  return 1;
}

// Row tiles of 128 instead of 192 rows (same waves, 32-row wave tiles) fill
// the CUs better at some row counts (1024 rows: 8 x 16 x 2 = 256 latent
// blocks, where 192-row tiles give 6 x 16 x 2 = 192 and leave most of the
// last tile empty), at a higher cost per output (measured at 1024 rows, K
// split in 2, one box: packed latent GEMM 54.1-54.6 against 63.4-63.5 us,
// router 49.6-50.2 against 55.2, for 2/3 of the work per block: 1.28 and
// 1.36 times the cost per output). A call takes 128-row tiles, with the K
// split that suits them, where a model of the GEMM's time predicts them 5 %
// faster than the 192-row plan above: rounds of 256 blocks times one
// block's time (its rows x K stages at the measured cost of its tile
// height; a 192-row block over the full K takes about 127 us in the latent
// GEMM and 105 in the router's) plus the combine pass of a K split (its
// partials at the combine kernels' measured rates). Every output is the
// same sum in the same order whatever the tile height; only the K split
// changes the order of the additions.
struct GemmPlan {
  int bm;  // block rows
  int ns;  // K splits
};

static double gemm_model_us(int rows, bool router, int bm, int ns) {
  const int nt = router ? kRouterCols / 192 : kLatent / 224;
  const double full_us = router ? 105.0 : 127.0;                   // 192-row block, full K
  const double per_out = bm == 192 ? 1.0 : (router ? 1.36 : 1.28);  // cost per output, relative
  const int blocks = (rows + bm - 1) / bm * nt * ns;
  const int rounds = (blocks + 255) / 256;
  double t = rounds * full_us * (bm / 192.0) * per_out / ns;
  if (ns > 1)
    t += router ? 1.0 + ns * (double)rows * kExperts * 8 / 3.5e6
                : 1.0 + (ns * (double)rows * kLatent * 4 + (double)rows * kLatent * 2) / 5.2e6;
  return t;
}

static GemmPlan prefill_gemm_plan(int rows, bool router, bool can_split) {
  const GemmPlan base{kGBM, can_split ? prefill_splits((rows + kGBM - 1) / kGBM, router) : 1};
  GemmPlan best = base;
  double t_best = 0.95 * gemm_model_us(rows, router, base.bm, base.ns);
  for (const int ns : {1, 2, 4, 7, 14}) {
    if (ns > 1 && !can_split) break;
    const double t = gemm_model_us(rows, router, 128, ns);
    if (t < t_best) {
      best = GemmPlan{128, ns};
      t_best = t;
    }
  }
  return best;
}

// Latent combine: latent[r][n] = BF16(sum over splits of part[q][r][n]), the
// sum in FP64 in split order, one rounding. 4 outputs per thread; the split
// count is a template argument so that every split's load is in flight
// before the first add.
template <int NS>
__global__ __launch_bounds__(256) void latent_combine_kernel(const float* __restrict__ part,
                                                             uint16_t* __restrict__ latent, int rows) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * (kLatent / 4)) return;
  const size_t plane = (size_t)rows * kLatent;
  f32x4 v[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) v[q] = *reinterpret_cast<const f32x4*>(part + q * plane + 4 * i);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int q = 0; q < NS; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += (double)v[q][c];
  u32x2 o;
  o[0] = (uint32_t)f64_to_bf16_rne(acc[0]) | ((uint32_t)f64_to_bf16_rne(acc[1]) << 16);
  o[1] = (uint32_t)f64_to_bf16_rne(acc[2]) | ((uint32_t)f64_to_bf16_rne(acc[3]) << 16);
  *reinterpret_cast<u32x2*>(latent + 4 * i) = o;
}

// Router combine: logits[r][e] = FP32(sum over splits of part[q][r][e]) in
// FP64 split order, then the exact recompute of any non-finite logit. One
// workgroup per 16 rows x 64 experts (enough workgroups to spread the
// partials' loads at one row tile); thread t sums row r0 + t / 16, experts
// e0 + 4 (t % 16) .. + 3.
constexpr int kCombRows = 16;

template <bool BT, int NS>
__global__ __launch_bounds__(256) void router_combine_kernel(const double* __restrict__ part,
                                                             float* __restrict__ logits, int rows,
                                                             const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ parts_w) {
  __shared__ uint64_t bad_rows;
  __shared__ double red[256];
  const int r0 = blockIdx.x * kCombRows;
  const int e0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int r = r0 + (t >> 4);
  bool bad = false;
  if (r < rows) {
    const size_t plane = (size_t)rows * kExperts;
    const double* src = part + (size_t)r * kExperts + e0 + 4 * (t & 15);
    f64x2 v[NS][2];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) v[q][h] = *reinterpret_cast<const f64x2*>(src + q * plane + 2 * h);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += v[q][c >> 1][c & 1];
    const f32x4 o = {(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
    *reinterpret_cast<f32x4*>(logits + (size_t)r * kExperts + e0 + 4 * (t & 15)) = o;
#pragma unroll
    for (int c = 0; c < 4; ++c) bad |= f32_nonfinite(o[c]);
  }
  if (t == 0) bad_rows = 0;
  __syncthreads();
  const uint64_t m = ballot(bad);    // lanes 16 j .. 16 j + 15 of wave w hold row 4 w + j
  if (lane == 0 && m != 0) {
    uint64_t mine = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((m >> (16 * j)) & 0xFFFFu) mine |= 1ull << (4 * wave + j);
    atomicOr((unsigned long long*)&bad_rows, (unsigned long long)mine);
  }
  __syncthreads();
  const uint64_t mask[1] = {bad_rows};
  if (mask[0] != 0) router_recompute<BT, 1>(x, parts_w, logits, r0, e0 / 64, mask, red);
}

// The three exact BF16 parts of an FP32 weight: each takes the top 8
// significant bits (nearest-even) of what the previous ones leave.
__device__ __forceinline__ void split3(float wv, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_rne(wv);
  const float r1 = wv - __uint_as_float(hi << 16);
  mid = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_rne(r2);
}

// Split the FP32 router weight into its three exact BF16 parts, stored as
// parts[k][e / 64][p][e % 64]. One thread per 8 consecutive experts of a row.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                           uint16_t* __restrict__ parts) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int k = t / (kExperts / 8);
  const int e = (t % (kExperts / 8)) * 8;
  if (k >= kHidden) return;
  const f32x4 v0 = __builtin_nontemporal_load((const f32x4*)(wr + (size_t)k * kExperts + e));
  const f32x4 v1 = __builtin_nontemporal_load((const f32x4*)(wr + (size_t)k * kExperts + e + 4));
  uint32_t p[3][4];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float wv = c < 4 ? v0[c] : v1[c - 4];
    uint32_t hi, mid, lo;
    split3(wv, hi, mid, lo);
    const int sh = (c & 1) * 16;
    if ((c & 1) == 0) p[0][c >> 1] = p[1][c >> 1] = p[2][c >> 1] = 0u;
    p[0][c >> 1] |= hi << sh;
    p[1][c >> 1] |= mid << sh;
    p[2][c >> 1] |= lo << sh;
  }
  uint16_t* dst = parts + (size_t)k * kRouterCols + (e / 64) * 192 + (e % 64);
#pragma unroll
  for (int q = 0; q < 3; ++q)
    *(u32x4*)(dst + 64 * q) = u32x4{p[q][0], p[q][1], p[q][2], p[q][3]};
}

// Packing for the K-contiguous GEMM variant, once per weight set, through
// 32 x 32 LDS tiles: W [7168][3584] -> WT [3584][7168]; Wr [7168][896] ->
// its three BF16 parts as partsT [2688][7168], part p of expert e in row
// (e / 64) * 192 + 64 p + e % 64 (the column order of the [K][N] parts).
__global__ __launch_bounds__(256) void pack_prefill_latent_kernel(const uint16_t* __restrict__ w,
                                                                  uint16_t* __restrict__ wt) {
  __shared__ uint16_t tile[32][34];
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) tile[ty + 8 * i][tx] = w[(size_t)(k0 + ty + 8 * i) * kLatent + n0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) wt[(size_t)(n0 + ty + 8 * i) * kHidden + k0 + tx] = tile[tx][ty + 8 * i];
}

__global__ __launch_bounds__(256) void pack_prefill_router_kernel(const float* __restrict__ wr,
                                                                  uint16_t* __restrict__ parts_t) {
  __shared__ float tile[32][33];
  const int e0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) tile[ty + 8 * i][tx] = wr[(size_t)(k0 + ty + 8 * i) * kExperts + e0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + ty + 8 * i;
    uint32_t p[3];
    split3(tile[tx][ty + 8 * i], p[0], p[1], p[2]);
#pragma unroll
    for (int q = 0; q < 3; ++q)
      parts_t[(size_t)((e / 64) * 192 + 64 * q + e % 64) * kHidden + k0 + tx] = (uint16_t)p[q];
  }
}

size_t prefill_packed_latent_bytes() { return (size_t)kLatent * kHidden * 2; }
size_t prefill_packed_bytes() { return prefill_packed_latent_bytes() + (size_t)kRouterCols * kHidden * 2; }

hipError_t launch_pack_prefill_weights(const uint16_t* w_latent, const float* w_router, void* packed,
                                       hipStream_t stream) {
  uint16_t* wt = static_cast<uint16_t*>(packed);
  uint16_t* parts_t = reinterpret_cast<uint16_t*>(static_cast<char*>(packed) + prefill_packed_latent_bytes());
  const hipError_t e = launch_kernel(pack_prefill_latent_kernel, dim3(kLatent / 32, kHidden / 32), dim3(256),
                                     stream, w_latent, wt);
  if (e != hipSuccess) return e;
  return launch_kernel(pack_prefill_router_kernel, dim3(kExperts / 32, kHidden / 32), dim3(256), stream,
                       w_router, parts_t);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Bytes of the K-split partials of a call of `rows` rows: the latent GEMM's
// FP32 and the router GEMM's FP64 sums per split, one after the other in
// time, so they share one area.
static size_t split_part_bytes(int rows) {
  const int sl = prefill_gemm_plan(rows, false, true).ns;
  const int sr = prefill_gemm_plan(rows, true, true).ns;
  const size_t lat = sl > 1 ? (size_t)sl * rows * kLatent * sizeof(float) : 0;
  const size_t rt = sr > 1 ? (size_t)sr * rows * kExperts * sizeof(double) : 0;
  return lat > rt ? lat : rt;
}

size_t prefill_workspace_bytes(int rows_cap, size_t* off_logits, size_t* off_parts, size_t* off_cand,
                               size_t* off_split) {
  *off_parts = 0;
  size_t off = align256(sizeof(uint16_t) * (size_t)kHidden * kRouterCols);
  *off_logits = off;
  off += align256(sizeof(float) * (size_t)rows_cap * kExperts);
  *off_cand = off;
  off += align256(sizeof(uint64_t) * (size_t)rows_cap * kTopkMaxShards * kTopK);
  *off_split = off;
  // the largest split area over every row count the plan accepts
  size_t most = 0;
  for (int r = 1; r <= rows_cap; ++r) {
    const size_t b = split_part_bytes(r);
    most = b > most ? b : most;
  }
  return off + align256(most);
}

// One GEMM over `rows` rows with `ns` K splits and `BM`-row tiles, then the
// combine of the split sums.
template <bool Router, bool BT, int BM>
static hipError_t launch_gemm_tiles(const uint16_t* x, const uint16_t* w, void* out, int rows, int ns,
                                    void* part, hipStream_t stream) {
  using S = GemmShape<Router, BM>;
  const int mt = (rows + BM - 1) / BM;
  const int blocks = mt * (S::N / S::BN) * ns;
  hipError_t e = launch_kernel(prefill_gemm_kernel<Router, BT, BM>, dim3(blocks), dim3(kGThreads), stream, x, w,
                               out, rows, mt, ns, ns > 1 ? part : nullptr);
  if (e != hipSuccess || ns == 1) return e;
  if constexpr (Router) {
    const dim3 grid((rows + kCombRows - 1) / kCombRows, kExperts / 64);
    const double* pp = static_cast<const double*>(part);
    float* lg = static_cast<float*>(out);
    switch (ns) {
      case 2: return launch_kernel(router_combine_kernel<BT, 2>, grid, dim3(256), stream, pp, lg, rows, x, w);
      case 4: return launch_kernel(router_combine_kernel<BT, 4>, grid, dim3(256), stream, pp, lg, rows, x, w);
      case 7: return launch_kernel(router_combine_kernel<BT, 7>, grid, dim3(256), stream, pp, lg, rows, x, w);
      case 14: return launch_kernel(router_combine_kernel<BT, 14>, grid, dim3(256), stream, pp, lg, rows, x, w);
      default: return hipErrorInvalidValue;
    }
  } else {
    const dim3 grid((unsigned)(((size_t)rows * (kLatent / 4) + 255) / 256));
    const float* pp = static_cast<const float*>(part);
    uint16_t* lt = static_cast<uint16_t*>(out);
    switch (ns) {
      case 2: return launch_kernel(latent_combine_kernel<2>, grid, dim3(256), stream, pp, lt, rows);
      case 4: return launch_kernel(latent_combine_kernel<4>, grid, dim3(256), stream, pp, lt, rows);
      case 7: return launch_kernel(latent_combine_kernel<7>, grid, dim3(256), stream, pp, lt, rows);
      case 14: return launch_kernel(latent_combine_kernel<14>, grid, dim3(256), stream, pp, lt, rows);
      default: return hipErrorInvalidValue;
    }
  }
}

// One GEMM over `rows` rows, K-split when `part` is given and the row tiles
// are few, with the tile height and split of prefill_gemm_plan.
template <bool Router, bool BT>
static hipError_t launch_gemm(const uint16_t* x, const uint16_t* w, void* out, int rows, void* part,
                              hipStream_t stream) {
  const GemmPlan p = prefill_gemm_plan(rows, Router, part != nullptr);
  return p.bm == 128 ? launch_gemm_tiles<Router, BT, 128>(x, w, out, rows, p.ns, part, stream)
                     : launch_gemm_tiles<Router, BT, 192>(x, w, out, rows, p.ns, part, stream);
}

static_assert(kGKT % (28 * kGFoldStages) == 0, "every split of the K stages is whole fold periods");

hipError_t launch_prefill_latent(const uint16_t* x, const uint16_t* w_latent, uint16_t* latent,
                                 int rows, void* part, hipStream_t stream) {
  if (rows < 1 || rows > kPrefillMaxRows) return hipErrorInvalidValue;
  return launch_gemm<false, false>(x, w_latent, latent, rows, part, stream);
}

hipError_t launch_prefill_packed(const uint16_t* x, const void* packed, uint16_t* latent, float* logits,
                                 int rows, void* part, hipStream_t stream) {
  if (rows < 1 || rows > kPrefillMaxRows) return hipErrorInvalidValue;
  const uint16_t* wt = static_cast<const uint16_t*>(packed);
  const uint16_t* parts_t =
      reinterpret_cast<const uint16_t*>(static_cast<const char*>(packed) + prefill_packed_latent_bytes());
  const hipError_t e = launch_gemm<false, true>(x, wt, latent, rows, part, stream);
  if (e != hipSuccess) return e;
  return launch_gemm<true, true>(x, parts_t, logits, rows, part, stream);
}

hipError_t launch_prefill_router(const uint16_t* x, const float* w_router, uint16_t* parts,
                                 float* logits, int rows, void* part, hipStream_t stream) {
  if (rows < 1 || rows > kPrefillMaxRows) return hipErrorInvalidValue;
  const hipError_t e = launch_kernel(router_split_kernel, dim3(kHidden * (kExperts / 8) / 256), dim3(256),
                                     stream, w_router, parts);
  if (e != hipSuccess) return e;
  return launch_gemm<true, false>(x, parts, logits, rows, part, stream);
}

}  // namespace route
