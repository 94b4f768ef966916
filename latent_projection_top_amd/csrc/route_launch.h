// Host-side launchers of the route kernels (called by the C ABI in route_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace route {

// Enqueue `kernel` on `stream` and return the status of this launch alone.
// hipLaunchKernel reports what went wrong with the launch itself; reading
// hipGetLastError() after a launch would instead return (and clear) an error
// left behind by unrelated earlier calls on the thread. The arguments are
// converted to the kernel's parameter types and kept alive for the call.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "one argument per kernel parameter");
  std::tuple<std::decay_t<Params>...> vals{static_cast<std::decay_t<Params>>(args)...};
  void* ptrs[sizeof...(Params) > 0 ? sizeof...(Params) : 1];
  std::apply([&ptrs](auto&... v) {
    size_t i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

// Decode workspace: tile counters, then split-K partials, then a logits buffer.
struct DecodeWorkspace {
  uint32_t* counters;  // kDecodeCounters entries, zero between calls
  float* lat_part;     // [kSplits][rows_cap][3584]
  double* rt_part;     // [kSplits][rows_cap][896]
};

// Decode output shapes: the whole route (3584, 896) or one tensor-parallel
// rank's share of it, (448, 112) at 8 ranks and (224, 56) at 16 ranks.
bool decode_shape_valid(int latent, int experts);
size_t decode_workspace_bytes(int rows_cap, int latent, int experts, size_t* off_lat, size_t* off_rt,
                              size_t* off_logits, size_t* off_cand);
size_t prefill_workspace_bytes(int rows_cap, size_t* off_logits, size_t* off_parts, size_t* off_cand,
                               size_t* off_split);

hipError_t launch_decode_route(const uint16_t* x, const uint16_t* w_latent, const float* w_router,
                               uint16_t* latent, float* logits, int32_t* ids, float* weights,
                               const DecodeWorkspace& ws, int rows, int rows_cap, int n_latent,
                               int n_experts, bool fuse_topk, bool packed, hipStream_t stream);

// Packed decode weights (whole route only): the latent weight's values
// reordered into the decode kernel's consumption order, followed by the router
// weight's, same byte counts as the [K][N] weights.
size_t decode_packed_latent_bytes();
size_t decode_packed_bytes();
hipError_t launch_pack_decode_weights(const uint16_t* w_latent, const float* w_router, void* packed,
                                      hipStream_t stream);

// Static device scratch of the allocation-free entry point (one per GPU).
// static_scratch_init takes the array's device address on `device` (made
// current for the call) and clears it, once per device; static_scratch
// returns that address (nullptr before a successful init) and its size.
// static_decode_workspace lays a decode workspace for up to 20 rows of the
// packed launches over it, with a logits buffer; from static_free_offset on,
// the array holds nothing a later call needs (partials and logits only).
hipError_t static_scratch_init(int device);
void* static_scratch(int device, size_t* bytes);
DecodeWorkspace static_decode_workspace(void* base, float** logits);
size_t static_free_offset();

hipError_t launch_topk16(const float* logits, int32_t* ids, float* weights, int rows,
                         hipStream_t stream);

// Sharded top-16 (stage 1: local top-16 per expert shard into cand
// [rows][shards][16] uint64 keys; stage 2: merge). shards divides 896 with at
// least 16 experts per shard, at most kTopkMaxShards.
constexpr int kTopkMaxShards = 56;
bool topk16_shards_valid(int shards);
hipError_t launch_topk16_sharded(const float* logits, int shards, int32_t* ids, float* weights,
                                 uint64_t* cand, int rows, hipStream_t stream);

// `part`: the workspace's K-split area, or NULL for launches that may not
// split (the allocation-free entry point).
hipError_t launch_prefill_latent(const uint16_t* x, const uint16_t* w_latent, uint16_t* latent,
                                 int rows, void* part, hipStream_t stream);

// parts: workspace for the three BF16 parts of w_router ([7168][2688] BF16)
hipError_t launch_prefill_router(const uint16_t* x, const float* w_router, uint16_t* parts,
                                 float* logits, int rows, void* part, hipStream_t stream);

// Packed prefill weights: W as [3584][7168] BF16, then the router weight's
// three exact BF16 parts as [2688][7168] (K contiguous); the GEMMs read them
// with the same per-lane operands as the [K][N] path.
size_t prefill_packed_latent_bytes();
size_t prefill_packed_bytes();
hipError_t launch_pack_prefill_weights(const uint16_t* w_latent, const float* w_router, void* packed,
                                       hipStream_t stream);
hipError_t launch_prefill_packed(const uint16_t* x, const void* packed, uint16_t* latent, float* logits,
                                 int rows, void* part, hipStream_t stream);

}  // namespace route
