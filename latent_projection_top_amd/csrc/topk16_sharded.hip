// Sharded top-16: the selection half of a route whose experts are split over
// ranks. Each of `shards` contiguous expert shards selects its local top-16;
// the 16 * shards candidates are then merged into the global top-16.
//
// Page "Kimi K3.1 recipe: route 9..20 decode rows through the pushed pair
// gather and standalone top-16" (voipmonitor/flare pull request 24), "What /
// why": the standalone top-16 selects 16 experts per row; page
// "Use two row blocks for eight-row Kimi paired gathers" (NVIDIA/hyperflare-
// inference pull request 265) gives the per-rank router output as 56 experts
// (16 ranks). The merge is exact: under one total order the global top 16
// lie in the union of the shards' local top 16s (a key with 16 larger keys in
// its own shard has at least 16 larger keys overall). Both stages use the
// same selection as topk16_wave, so the result is bitwise that of
// route_topk16.
#include "route_device.h"
#include "route_launch.h"

namespace route {

constexpr int kShardRowsPerBlock = 4;  // one wave per (row, shard) or per row

// Stage 1: wave (row, shard) selects the 16 largest keys of experts
// shard * S .. shard * S + S - 1 (keys carry the global expert index).
template <int P>
__global__ __launch_bounds__(kWave * kShardRowsPerBlock) void topk16_shard_kernel(
    const float* __restrict__ logits, uint64_t* __restrict__ cand, int rows, int shards) {
  __shared__ uint64_t scratch[kShardRowsPerBlock][kTopkScratch];
  const int item = blockIdx.x * kShardRowsPerBlock + (threadIdx.x >> 6);
  if (item >= rows * shards) return;  // whole waves leave together
  const int row = item / shards;
  const int shard = item % shards;
  const int size = kExperts / shards;
  const int lane = threadIdx.x & (kWave - 1);
  const float* lg = logits + (size_t)row * kExperts;
  uint64_t c[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int j = i * kWave + lane;
    c[i] = j < size ? select_key<false>(lg, (uint32_t)(shard * size + j)) : 0ull;
  }
  const uint64_t k = select16<P>(c, scratch[threadIdx.x >> 6]);
  if (lane < kTopK) cand[(size_t)item * kTopK + lane] = k;
}

// Stage 2: wave `row` selects the 16 largest of the row's 16 * shards
// candidates and writes ids and weights.
template <int Q>
__global__ __launch_bounds__(kWave * kShardRowsPerBlock) void topk16_merge_kernel(
    const uint64_t* __restrict__ cand, int32_t* __restrict__ ids, float* __restrict__ weights,
    int rows, int shards) {
  __shared__ uint64_t scratch[kShardRowsPerBlock][kTopkScratch];
  const int row = blockIdx.x * kShardRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int n = kTopK * shards;
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t* cr = cand + (size_t)row * n;
  uint64_t c[Q];
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const int j = i * kWave + lane;
    c[i] = j < n ? cr[j] : 0ull;
  }
  write_selection(select16<Q>(c, scratch[threadIdx.x >> 6]), ids + (size_t)row * kTopK,
                  weights + (size_t)row * kTopK);
}

bool topk16_shards_valid(int shards) {
  return shards >= 1 && shards <= kTopkMaxShards && kExperts % shards == 0 &&
         kExperts / shards >= kTopK;
}

template <int P>
static hipError_t launch_stage1(const float* logits, uint64_t* cand, int rows, int shards, hipStream_t s) {
  const int blocks = (rows * shards + kShardRowsPerBlock - 1) / kShardRowsPerBlock;
  return launch_kernel(topk16_shard_kernel<P>, dim3(blocks), dim3(kWave * kShardRowsPerBlock), s, logits,
                       cand, rows, shards);
}

template <int Q>
static hipError_t launch_stage2(const uint64_t* cand, int32_t* ids, float* weights, int rows, int shards,
                                hipStream_t s) {
  const int blocks = (rows + kShardRowsPerBlock - 1) / kShardRowsPerBlock;
  return launch_kernel(topk16_merge_kernel<Q>, dim3(blocks), dim3(kWave * kShardRowsPerBlock), s, cand, ids,
                       weights, rows, shards);
}

hipError_t launch_topk16_sharded(const float* logits, int shards, int32_t* ids, float* weights,
                                 uint64_t* cand, int rows, hipStream_t stream) {
  if (!topk16_shards_valid(shards) || rows < 1) return hipErrorInvalidValue;
  // keys per lane: stage 1 holds one shard, stage 2 the 16 * shards candidates
  // both stages' template variants are chosen before anything is launched
  const int p = (kExperts / shards + kWave - 1) / kWave;
  const int q = (kTopK * shards + kWave - 1) / kWave;
  if ((p != 1 && p != 2 && p != 4 && p != 7 && p != 14) ||
      (q != 1 && q != 2 && q != 4 && q != 7 && q != 8 && q != 14))
    return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  switch (p) {
    case 1: e = launch_stage1<1>(logits, cand, rows, shards, stream); break;
    case 2: e = launch_stage1<2>(logits, cand, rows, shards, stream); break;
    case 4: e = launch_stage1<4>(logits, cand, rows, shards, stream); break;
    case 7: e = launch_stage1<7>(logits, cand, rows, shards, stream); break;
    default: e = launch_stage1<14>(logits, cand, rows, shards, stream); break;
  }
  if (e != hipSuccess) return e;
  switch (q) {
    case 1: return launch_stage2<1>(cand, ids, weights, rows, shards, stream);
    case 2: return launch_stage2<2>(cand, ids, weights, rows, shards, stream);
    case 4: return launch_stage2<4>(cand, ids, weights, rows, shards, stream);
    case 7: return launch_stage2<7>(cand, ids, weights, rows, shards, stream);
    case 8: return launch_stage2<8>(cand, ids, weights, rows, shards, stream);
    default: return launch_stage2<14>(cand, ids, weights, rows, shards, stream);
  }
}

}  // namespace route
