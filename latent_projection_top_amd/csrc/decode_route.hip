// Decode route (1..20 rows): latent down projection + FP32 router logits in one
// weight-streaming, split-K kernel, with the standalone top-16 optionally
// fused into its epilogue.
//
// What is computed (page "Optionally gather the Kimi3 prefill latent instead of
// reducing it", voipmonitor/flare pull request 16, Description, numerics
// bullet): every latent value is one FP32-accumulated dot product over the
// full K = 7168, rounded to BF16 once. On one GPU there is no exchange: the K
// range is split S = 8 ways only to spread the 77 MB of weights over all
// compute units, and the S partials are combined in FP64 in a fixed order
// before the single rounding.
//
// Shape of the work (all constants, K = 7168, N = 3584, E = 896):
//   latent blocks: 56 column tiles of 64 x 8 K-splits of 896 rows = 448 blocks
//   router blocks: 28 expert tiles of 32 x 8 K-splits of 896 rows = 224 blocks
// Every block streams the same 114,688 bytes of weight (896 rows x 128 bytes),
// so the 672 blocks finish together. Four waves per block take 224 rows each.
//
// Latent, per wave and 32-row step: each lane reads 8 rows x 4 columns
// (8-byte loads; 16 lanes cover one 128-byte row segment), transposes the 8x4
// BF16 block in registers with v_perm so that each of 4 registers holds 8
// consecutive-K values of one column, and issues 4 (or 8 for 17..20 rows)
// v_mfma_f32_16x16x32_bf16 with the hidden rows as the 16-wide N side. The MFMA
// accumulates in FP32. Rows are padded to 16 (32) inside the MFMA only.
//
// Router, per wave: v_mfma_f64_16x16x4_f64 with FP32 weights widened to FP64
// (exact) and BF16 hidden values widened to FP64 (exact): the logits are
// accumulated in FP64 end to end and rounded to FP32 once.
//
// Split-K combine: each block sums its 4 waves (FP64, fixed order) and stores
// one partial per output (latent: FP32, router: FP64). The last of a tile's 8
// blocks (integer counter, release/acquire fences) sums the 8 partials in FP64
// in split order, rounds once, writes the output and resets the counter. With
// fuse_topk the last router tile to finish then runs the top-16 for every row.
#include "route_device.h"
#include "route_launch.h"

namespace route {

constexpr int kSplits = 8;
constexpr int kKSplit = kHidden / kSplits;           // 896
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;             // 256
constexpr int kKWave = kKSplit / kWaves;             // 224
constexpr int kStep = 32;
constexpr int kStepsPerWave = kKWave / kStep;        // 7
constexpr int kLatTileN = 64;
constexpr int kLatTiles = kLatent / kLatTileN;       // 56
constexpr int kRtTileE = 32;
constexpr int kRtTiles = kExperts / kRtTileE;        // 28
constexpr int kLatBlocks = kLatTiles * kSplits;      // 448
constexpr int kRtBlocks = kRtTiles * kSplits;        // 224
constexpr int kDecodeBlocks = kLatBlocks + kRtBlocks;
constexpr int kDecodeCounters = kLatTiles + kRtTiles + 1;
constexpr int kDecodeMaxRows = 20;

static_assert(kHidden % (kSplits * kWaves * kStep) == 0, "K split");
static_assert(kLatent % kLatTileN == 0 && kExperts % kRtTileE == 0, "tiles");

struct DecodeArgs {
  const uint16_t* __restrict__ x;
  const uint16_t* __restrict__ w;
  const float* __restrict__ wr;
  uint16_t* __restrict__ latent;
  float* __restrict__ logits;
  int32_t* __restrict__ ids;
  float* __restrict__ weights;
  float* __restrict__ lat_part;
  double* __restrict__ rt_part;
  uint32_t* __restrict__ counters;
  int rows;
  int rows_cap;
  int fuse_topk;
};

// Cross-workgroup handoff without device-wide cache maintenance. Each XCD has
// its own L2 and a device-scope fence would write back and invalidate the whole
// L2 for every workgroup. Instead, everything one workgroup hands to another
// (partials, logits for the fused select, counters) moves through device-scope
// relaxed atomic stores and loads, which the compiler emits with the sc1 bit so
// that they are coherent across XCDs; a store is complete once vmcnt drains.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's outstanding vector memory operations (stores
// included: GFX9 counts them in vmcnt) have completed.
__device__ __forceinline__ void drain_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// True in the workgroup that arrives last of `expected`. Every thread's st_dev
// stores are complete before thread 0 bumps the counter, so the last workgroup
// reads all of them with ld_dev.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, int expected, int* flag) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (prev == (uint32_t)(expected - 1));
  }
  __syncthreads();
  return *flag != 0;
}

template <int NT>
__device__ void latent_block(const DecodeArgs& a, int b, float* red, int* flag) {
  const int tile = b % kLatTiles;
  const int split = b / kLatTiles;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int m = lane & 15;
  const int n0 = tile * kLatTileN;
  const int k0 = split * kKSplit + wave * kKWave;

  f32x4 acc[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[nt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* wp = a.w + (size_t)(k0 + 8 * g) * kLatent + n0 + 4 * m;
  const uint16_t* xp[NT];
  bool xok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 16 * nt + m;
    xok[nt] = r < a.rows;
    xp[nt] = a.x + (size_t)(xok[nt] ? r : 0) * kHidden + k0 + 8 * g;
  }

#pragma unroll
  for (int st = 0; st < kStepsPerWave; ++st) {
    u32x2 wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wv[j] = __builtin_nontemporal_load((const u32x2*)(wp + (size_t)(st * kStep + j) * kLatent));
    u32x4 xv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      xv[nt] = xok[nt] ? *(const u32x4*)(xp[nt] + st * kStep) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 av;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        av[p] = __builtin_amdgcn_perm(wv[2 * p + 1][c >> 1], wv[2 * p][c >> 1], sel);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, xv[nt]), acc[nt][c], 0, 0, 0);
    }
  }

  // lane (g, m) holds row 16*nt + m, local columns 16*g + 4*t + c
  constexpr int kRowsPad = 16 * NT;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        red[(wave * kRowsPad + 16 * nt + m) * kLatTileN + 16 * g + 4 * t + c] = acc[nt][c][t];
  __syncthreads();

  const int outs = a.rows * kLatTileN;
  for (int i = threadIdx.x; i < outs; i += kThreads) {
    const int r = i / kLatTileN;
    const int col = i % kLatTileN;
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += (double)red[(w * kRowsPad + r) * kLatTileN + col];
    st_dev(&a.lat_part[((size_t)split * a.rows_cap + r) * kLatent + n0 + col], (float)s);
  }

  if (!last_arrival(&a.counters[tile], kSplits, flag)) return;

  for (int i = threadIdx.x; i < outs; i += kThreads) {
    const int r = i / kLatTileN;
    const int col = i % kLatTileN;
    double s = 0.0;
#pragma unroll
    for (int sp = 0; sp < kSplits; ++sp)
      s += (double)ld_dev(&a.lat_part[((size_t)sp * a.rows_cap + r) * kLatent + n0 + col]);
    a.latent[(size_t)r * kLatent + n0 + col] = f64_to_bf16_rne(s);
  }
  if (threadIdx.x == 0) st_dev(&a.counters[tile], 0u);
}

template <int NT>
__device__ void router_block(const DecodeArgs& a, int b, double* red, int* flag) {
  const int tile = b % kRtTiles;
  const int split = b / kRtTiles;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int m = lane & 15;
  const int e0 = tile * kRtTileE;
  const int k0 = split * kKSplit + wave * kKWave;

  f64x4 acc[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[nt][c] = f64x4{0.0, 0.0, 0.0, 0.0};

  const float* wp = a.wr + (size_t)(k0 + 8 * g) * kExperts + e0 + 2 * m;
  const uint16_t* xp[NT];
  bool xok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 16 * nt + m;
    xok[nt] = r < a.rows;
    xp[nt] = a.x + (size_t)(xok[nt] ? r : 0) * kHidden + k0 + 8 * g;
  }

#pragma unroll 1
  for (int st = 0; st < kStepsPerWave; ++st) {
    f32x2 wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wv[j] = __builtin_nontemporal_load((const f32x2*)(wp + (size_t)(st * kStep + j) * kExperts));
    double xd[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 xv = xok[nt] ? *(const u32x4*)(xp[nt] + st * kStep) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        xd[nt][2 * p] = (double)bf16_lo(xv[p]);
        xd[nt][2 * p + 1] = (double)bf16_hi(xv[p]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double w0 = (double)wv[j][0];
      const double w1 = (double)wv[j][1];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(w0, xd[nt][j], acc[nt][0], 0, 0, 0);
        acc[nt][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(w1, xd[nt][j], acc[nt][1], 0, 0, 0);
      }
    }
  }

  // The FP64 MFMA keeps D[4*t + g][m] in slot t of lane (g, m): lane (g, m)
  // holds row 16*nt + m, local experts 2*(4*t + g) + c = 8*t + 2*g + c.
  constexpr int kRowsPad = 16 * NT;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        red[(wave * kRowsPad + 16 * nt + m) * kRtTileE + 8 * t + 2 * g + c] = acc[nt][c][t];
  __syncthreads();

  const int outs = a.rows * kRtTileE;
  for (int i = threadIdx.x; i < outs; i += kThreads) {
    const int r = i / kRtTileE;
    const int e = i % kRtTileE;
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[(w * kRowsPad + r) * kRtTileE + e];
    st_dev(&a.rt_part[((size_t)split * a.rows_cap + r) * kExperts + e0 + e], s);
  }

  if (!last_arrival(&a.counters[kLatTiles + tile], kSplits, flag)) return;

  for (int i = threadIdx.x; i < outs; i += kThreads) {
    const int r = i / kRtTileE;
    const int e = i % kRtTileE;
    double s = 0.0;
#pragma unroll
    for (int sp = 0; sp < kSplits; ++sp) s += ld_dev(&a.rt_part[((size_t)sp * a.rows_cap + r) * kExperts + e0 + e]);
    st_dev(&a.logits[(size_t)r * kExperts + e0 + e], (float)s);
  }
  if (threadIdx.x == 0) st_dev(&a.counters[kLatTiles + tile], 0u);

  if (!a.fuse_topk) return;
  uint32_t* done = &a.counters[kLatTiles + kRtTiles];
  if (!last_arrival(done, kRtTiles, flag)) return;
  for (int r = wave; r < a.rows; r += kWaves)
    topk16_wave<true>(a.logits + (size_t)r * kExperts, a.ids + (size_t)r * kTopK,
                      a.weights + (size_t)r * kTopK);
  if (threadIdx.x == 0) st_dev(done, 0u);
}

template <int NT>
__global__ __launch_bounds__(kThreads) void decode_route_kernel(DecodeArgs a) {
  constexpr int kLatBytes = kWaves * 16 * NT * kLatTileN * 4;
  constexpr int kRtBytes = kWaves * 16 * NT * kRtTileE * 8;
  constexpr int kBytes = kLatBytes > kRtBytes ? kLatBytes : kRtBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];
  __shared__ int flag;
  const int b = blockIdx.x;
  if (b < kLatBlocks)
    latent_block<NT>(a, b, reinterpret_cast<float*>(smem), &flag);
  else
    router_block<NT>(a, b - kLatBlocks, reinterpret_cast<double*>(smem), &flag);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(int rows_cap, size_t* off_lat, size_t* off_rt, size_t* off_logits) {
  size_t off = align256(sizeof(uint32_t) * kDecodeCounters);
  *off_lat = off;
  off = align256(off + sizeof(float) * kSplits * (size_t)rows_cap * kLatent);
  *off_rt = off;
  off = align256(off + sizeof(double) * kSplits * (size_t)rows_cap * kExperts);
  *off_logits = off;
  off = align256(off + sizeof(float) * (size_t)rows_cap * kExperts);
  return off;
}

hipError_t launch_decode_route(const uint16_t* x, const uint16_t* w_latent, const float* w_router,
                               uint16_t* latent, float* logits, int32_t* ids, float* weights,
                               const DecodeWorkspace& ws, int rows, int rows_cap, bool fuse_topk,
                               hipStream_t stream) {
  if (rows < 1 || rows > kDecodeMaxRows || rows > rows_cap) return hipErrorInvalidValue;
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
  if (rows <= 16)
    hipLaunchKernelGGL(decode_route_kernel<1>, dim3(kDecodeBlocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_route_kernel<2>, dim3(kDecodeBlocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace route
