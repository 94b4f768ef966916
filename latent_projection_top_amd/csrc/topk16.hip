// Standalone top-16 over FP32 router logits: one wave per row.
//
// Page "Kimi K3.1 recipe: route 9..20 decode rows through the pushed pair
// gather and standalone top-16" (voipmonitor/flare pull request 24),
// "What / why": rounds of 9..20 rows select their experts with a standalone
// top-16 instead of the fused select; the same kernel serves prefill chunks.
#include "route_device.h"
#include "route_launch.h"

namespace route {

constexpr int kTopkRowsPerBlock = 4;

__global__ __launch_bounds__(kWave * kTopkRowsPerBlock) void topk16_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ weights,
    int rows) {
  __shared__ uint64_t scratch[kTopkRowsPerBlock][kTopkScratch];
  const int row = blockIdx.x * kTopkRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves leave together
  topk16_wave(logits + (size_t)row * kExperts, ids + (size_t)row * kTopK,
              weights + (size_t)row * kTopK, scratch[threadIdx.x >> 6]);
}

hipError_t launch_topk16(const float* logits, int32_t* ids, float* weights, int rows,
                         hipStream_t stream) {
  const int blocks = (rows + kTopkRowsPerBlock - 1) / kTopkRowsPerBlock;
  return launch_kernel(topk16_kernel, dim3(blocks), dim3(kWave * kTopkRowsPerBlock), stream, logits, ids,
                       weights, rows);
}

}  // namespace route
