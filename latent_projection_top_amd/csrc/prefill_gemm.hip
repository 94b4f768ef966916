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
// Latent: C[M][3584] = x[M][7168] * W[7168][3584], BF16 MFMA
// (v_mfma_f32_16x16x32_bf16), FP32 accumulation over all of K in the MFMA
// accumulators, one nearest-even rounding to BF16 at the end.
//
// Router: logits[M][896] = x * Wr with Wr in FP32. Each FP32 weight is split
// exactly into three BF16 parts (w = hi + mid + lo: each step takes the top 8
// significant bits of what is left; the remainder after two steps has at most
// 8 significant bits). x is BF16, so every product x*part is exact in FP32 and
// the contraction runs on the BF16 MFMA at three times the latent's work per
// weight. Every 32-wide K slice is summed by three MFMAs into a zeroed FP32
// accumulator and folded into FP64 accumulators; the logits are the FP64 sums
// rounded once to FP32.
//
// Operand staging: x tiles are K-contiguous and go to LDS as they are. W is
// stored [K][N] (N contiguous) while the MFMA wants 8 consecutive K values of
// one column per lane, so each thread transposes the 2 x 8 block it loaded
// (v_perm on BF16 pairs) and writes K-contiguous columns to LDS. Block tile
// 128 x 128, 4 waves of 64 x 64, BK = 32, two LDS stages.
#include "route_device.h"
#include "route_launch.h"

namespace route {

constexpr int kPBM = 128;
constexpr int kPBN = 128;
constexpr int kPBK = 32;
constexpr int kPThreads = 256;
constexpr int kPLd = kPBK + 8;  // LDS row stride in BF16 elements (80 bytes)
constexpr int kPrefillMaxRows = 3072;

static_assert(kHidden % kPBK == 0 && kLatent % kPBN == 0 && kExperts % kPBN == 0, "tiles");

// Split an FP32 value into three BF16 parts whose sum is exact.
__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_rne(w);
  const float r1 = w - __uint_as_float(hi << 16);
  mid = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_rne(r2);
}

template <int P>
struct PrefillSmem {
  uint16_t a[2][kPBM * kPLd];
  uint16_t b[2][P][kPBN * kPLd];
};

// Router == false: W is BF16 [K][N], output BF16. Router == true: W is FP32
// [K][N], output FP32.
template <bool Router>
__global__ __launch_bounds__(kPThreads) void prefill_gemm_kernel(const uint16_t* __restrict__ x,
                                                                 const void* __restrict__ wv,
                                                                 void* __restrict__ out, int rows,
                                                                 int n_total) {
  constexpr int P = Router ? 3 : 1;
  __shared__ PrefillSmem<P> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int m = lane & 15;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int nbn = n_total / kPBN;
  const int bn0 = (blockIdx.x % nbn) * kPBN;
  const int bm0 = (blockIdx.x / nbn) * kPBM;

  // A loads: 128 rows x 4 chunks of 8 -> 2 chunks per thread.
  int a_row[2], a_k[2];
  bool a_ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * kPThreads;
    a_row[i] = c >> 2;
    a_k[i] = (c & 3) * 8;
    a_ok[i] = bm0 + a_row[i] < rows;
  }
  // B loads: 16 row pairs x 16 column groups of 8 -> one 2 x 8 block per thread.
  const int b_k = (tid >> 4) * 2;
  const int b_n = (tid & 15) * 8;

  u32x4 ra[2];
  u32x4 rb16[2];          // BF16: rows b_k, b_k+1, 8 columns each
  float rb32[2][8];       // FP32: rows b_k, b_k+1, 8 columns each

  auto load_tile = [&](int kt) {
    const int k0 = kt * kPBK;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = a_ok[i] ? *(const u32x4*)(x + (size_t)(bm0 + a_row[i]) * kHidden + k0 + a_k[i])
                      : u32x4{0u, 0u, 0u, 0u};
    if constexpr (!Router) {
      const uint16_t* w = static_cast<const uint16_t*>(wv);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        rb16[r] = __builtin_nontemporal_load(
            (const u32x4*)(w + (size_t)(k0 + b_k + r) * n_total + bn0 + b_n));
    } else {
      const float* w = static_cast<const float*>(wv);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const f32x4 v0 = __builtin_nontemporal_load(
            (const f32x4*)(w + (size_t)(k0 + b_k + r) * n_total + bn0 + b_n));
        const f32x4 v1 = __builtin_nontemporal_load(
            (const f32x4*)(w + (size_t)(k0 + b_k + r) * n_total + bn0 + b_n + 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rb32[r][q] = v0[q];
          rb32[r][4 + q] = v1[q];
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *(u32x4*)(&sm.a[buf][a_row[i] * kPLd + a_k[i]]) = ra[i];
    if constexpr (!Router) {
      // column c of the 2 x 8 block: (row b_k, row b_k+1) as one BF16 pair
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t v = __builtin_amdgcn_perm(rb16[1][c >> 1], rb16[0][c >> 1], sel);
        *(uint32_t*)(&sm.b[buf][0][(b_n + c) * kPLd + b_k]) = v;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t h0, m0, l0, h1, m1, l1;
        split3(rb32[0][c], h0, m0, l0);
        split3(rb32[1][c], h1, m1, l1);
        *(uint32_t*)(&sm.b[buf][0][(b_n + c) * kPLd + b_k]) = h0 | (h1 << 16);
        *(uint32_t*)(&sm.b[buf][1][(b_n + c) * kPLd + b_k]) = m0 | (m1 << 16);
        *(uint32_t*)(&sm.b[buf][2][(b_n + c) * kPLd + b_k]) = l0 | (l1 << 16);
      }
    }
  };

  f32x4 acc[4][4];
  double acc64[Router ? 4 : 1][Router ? 4 : 1][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (Router) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc64[i][j][t] = 0.0;
  }

  constexpr int KT = kHidden / kPBK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    bf16x8 af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *(const bf16x8*)(&sm.a[buf][(wm * 64 + 16 * i + m) * kPLd + 8 * g]);
    if constexpr (!Router) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 bfr = *(const bf16x8*)(&sm.b[buf][0][(wn * 64 + 16 * j + m) * kPLd + 8 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = (wn * 64 + 16 * j + m) * kPLd + 8 * g;
        const bf16x8 bl = *(const bf16x8*)(&sm.b[buf][2][off]);
        const bf16x8 bmid = *(const bf16x8*)(&sm.b[buf][1][off]);
        const bf16x8 bh = *(const bf16x8*)(&sm.b[buf][0][off]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 t4 = f32x4{0.f, 0.f, 0.f, 0.f};
          t4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bl, t4, 0, 0, 0);
          t4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bmid, t4, 0, 0, 0);
          t4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bh, t4, 0, 0, 0);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc64[i][j][t] += (double)t4[t];
        }
      }
    }
    if (kt + 1 < KT) store_tile(buf ^ 1);
    __syncthreads();
  }

  // lane (g, m) of tile (i, j) holds row 16 i + 4 g + t, column 16 j + m
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = bm0 + wm * 64 + 16 * i + 4 * g + t;
      if (row >= rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = bn0 + wn * 64 + 16 * j + m;
        if constexpr (!Router)
          static_cast<uint16_t*>(out)[(size_t)row * n_total + col] = f32_to_bf16_rne(acc[i][j][t]);
        else
          static_cast<float*>(out)[(size_t)row * n_total + col] = (float)acc64[i][j][t];
      }
    }
  }
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t prefill_workspace_bytes(int rows_cap, size_t* off_logits) {
  *off_logits = 0;
  return align256(sizeof(float) * (size_t)rows_cap * kExperts);
}

hipError_t launch_prefill_latent(const uint16_t* x, const uint16_t* w_latent, uint16_t* latent,
                                 int rows, hipStream_t stream) {
  if (rows < 1 || rows > kPrefillMaxRows) return hipErrorInvalidValue;
  const int mb = (rows + kPBM - 1) / kPBM;
  hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3(mb * (kLatent / kPBN)), dim3(kPThreads), 0,
                     stream, x, (const void*)w_latent, (void*)latent, rows, kLatent);
  return hipGetLastError();
}

hipError_t launch_prefill_router(const uint16_t* x, const float* w_router, float* logits, int rows,
                                 hipStream_t stream) {
  if (rows < 1 || rows > kPrefillMaxRows) return hipErrorInvalidValue;
  const int mb = (rows + kPBM - 1) / kPBM;
  hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3(mb * (kExperts / kPBN)), dim3(kPThreads), 0,
                     stream, x, (const void*)w_router, (void*)logits, rows, kExperts);
  return hipGetLastError();
}

}  // namespace route
