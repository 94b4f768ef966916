// C ABI of the route library (libroute.so): plan preparation, argument checks
// and kernel launches. Every check runs before any launch; nothing allocates
// device memory or synchronises.
#include "route.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <new>

#include "route_launch.h"

struct route_plan {
  int32_t mode;
  int32_t rows_cap;
  int32_t device;
  int32_t latent;     // output shape: the whole route or one rank's share
  int32_t experts;
  size_t ws_bytes;
  size_t off_lat;     // decode: latent partials
  size_t off_rt;      // decode: router partials
  size_t off_logits;  // logits buffer for route_fused with logits == NULL
  size_t off_parts;   // prefill: BF16 parts of the router weight
  size_t off_cand;    // sharded top-16 candidates
  size_t off_split;   // prefill: K-split partials of chunks with few row tiles
};

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_device(const route_plan* p) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != p->device) return ROUTE_E_DEVICE;
  return ROUTE_OK;
}

int check_rows(const route_plan* p, int32_t rows) {
  return (rows < 1 || rows > p->rows_cap) ? ROUTE_E_ROWS : ROUTE_OK;
}

// A share plan (one tensor-parallel rank's columns) has no top-16: its
// experts are a fraction of the route's.
bool is_share(const route_plan* p) { return p->latent != ROUTE_LATENT || p->experts != ROUTE_EXPERTS; }

int status_of(hipError_t e) { return e == hipSuccess ? ROUTE_OK : ROUTE_E_HIP; }

route::DecodeWorkspace decode_ws(const route_plan* p, void* ws) {
  char* base = static_cast<char*>(ws);
  route::DecodeWorkspace d;
  d.counters = reinterpret_cast<uint32_t*>(base);
  d.lat_part = reinterpret_cast<float*>(base + p->off_lat);
  d.rt_part = reinterpret_cast<double*>(base + p->off_rt);
  return d;
}

int run_prefill_packed(const void* x, const void* packed, void* latent, float* logits, int32_t* ids,
                       float* weights, int32_t rows, bool fused, void* split, hipStream_t s) {
  int st = status_of(route::launch_prefill_packed(static_cast<const uint16_t*>(x), packed,
                                                  static_cast<uint16_t*>(latent), logits, rows, split, s));
  if (st != ROUTE_OK || !fused) return st;
  return status_of(route::launch_topk16(logits, ids, weights, rows, s));
}

int run_latent_router(const route_plan* p, const void* x, const void* w_latent, const float* w_router,
                      void* latent, float* logits, int32_t* ids, float* weights, void* ws,
                      int32_t rows, bool fused, hipStream_t s, bool packed = false) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (packed && p->mode == ROUTE_MODE_PREFILL)
    return run_prefill_packed(x, w_latent, latent, logits, ids, weights, rows, fused,
                              static_cast<char*>(ws) + p->off_split, s);
  const uint16_t* wb = static_cast<const uint16_t*>(w_latent);
  uint16_t* lb = static_cast<uint16_t*>(latent);
  if (p->mode == ROUTE_MODE_DECODE) {
    // decode: one launch; the fused select runs inside the projection kernel
    return status_of(route::launch_decode_route(xb, wb, w_router, lb, logits, ids, weights,
                                                decode_ws(p, ws), rows, p->rows_cap, p->latent,
                                                p->experts, fused, packed, s));
  }
  void* split = static_cast<char*>(ws) + p->off_split;
  int st = status_of(route::launch_prefill_latent(xb, wb, lb, rows, split, s));
  if (st != ROUTE_OK) return st;
  uint16_t* parts = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p->off_parts);
  st = status_of(route::launch_prefill_router(xb, w_router, parts, logits, rows, split, s));
  if (st != ROUTE_OK || !fused) return st;
  return status_of(route::launch_topk16(logits, ids, weights, rows, s));
}

// Packed weights serve whole-route plans (decode and prefill have their own
// formats); a rank share has none.
bool packed_plan(const route_plan* p) { return !is_share(p); }

size_t packed_bytes(const route_plan* p) {
  return p->mode == ROUTE_MODE_DECODE ? route::decode_packed_bytes() : route::prefill_packed_bytes();
}

// The decode packed buffer: latent values first, router values after them.
// (The prefill GEMM launcher splits its own buffer.)
const float* packed_router(const route_plan* p, const void* packed) {
  if (p->mode != ROUTE_MODE_DECODE) return nullptr;
  return reinterpret_cast<const float*>(static_cast<const char*>(packed) +
                                        route::decode_packed_latent_bytes());
}

}  // namespace

extern "C" {

int route_prepare(const route_config* cfg, route_plan** out) {
  if (out == nullptr) return ROUTE_E_ARG;
  *out = nullptr;
  if (cfg == nullptr || cfg->abi_version != ROUTE_ABI_VERSION) return ROUTE_E_ARG;
  if (cfg->mode != ROUTE_MODE_DECODE && cfg->mode != ROUTE_MODE_PREFILL) return ROUTE_E_ARG;
  if (cfg->hidden != ROUTE_HIDDEN || cfg->topk != ROUTE_TOPK ||
      !route::decode_shape_valid(cfg->latent, cfg->experts))
    return ROUTE_E_SHAPE;
  // rank shares are decode-only
  if (cfg->mode != ROUTE_MODE_DECODE && (cfg->latent != ROUTE_LATENT || cfg->experts != ROUTE_EXPERTS))
    return ROUTE_E_SHAPE;
  const int32_t max_rows = cfg->mode == ROUTE_MODE_DECODE ? ROUTE_DECODE_MAX_ROWS : ROUTE_PREFILL_MAX_ROWS;
  if (cfg->rows < 1 || cfg->rows > max_rows) return ROUTE_E_ROWS;

  int count = 0;
  if (cfg->device < 0 || hipGetDeviceCount(&count) != hipSuccess || cfg->device >= count)
    return ROUTE_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, cfg->device) != hipSuccess) return ROUTE_E_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return ROUTE_E_DEVICE;

  // the allocation-free entry point's static scratch: its device address is
  // taken (and the array cleared) once per device, here, with the device
  // current; a failure only disables that entry point on the device
  (void)route::static_scratch_init(cfg->device);

  route_plan* p = new (std::nothrow) route_plan();
  if (p == nullptr) return ROUTE_E_ARG;
  p->mode = cfg->mode;
  p->rows_cap = cfg->rows;
  p->device = cfg->device;
  p->latent = cfg->latent;
  p->experts = cfg->experts;
  if (p->mode == ROUTE_MODE_DECODE) {
    p->ws_bytes = route::decode_workspace_bytes(p->rows_cap, p->latent, p->experts, &p->off_lat,
                                                &p->off_rt, &p->off_logits, &p->off_cand);
    p->off_parts = p->off_split = 0;
  } else {
    p->off_lat = p->off_rt = 0;
    p->ws_bytes = route::prefill_workspace_bytes(p->rows_cap, &p->off_logits, &p->off_parts, &p->off_cand,
                                                 &p->off_split);
  }
  *out = p;
  return ROUTE_OK;
}

size_t route_workspace_bytes(const route_plan* plan) { return plan ? plan->ws_bytes : 0; }

int route_latent_router(const route_plan* plan, const void* x, const void* w_latent,
                        const float* w_router, void* latent, float* logits, void* workspace,
                        int32_t rows, void* stream) {
  if (!plan || !x || !w_latent || !w_router || !latent || !logits || !workspace) return ROUTE_E_ARG;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(x) || misaligned(w_latent) || misaligned(w_router) || misaligned(latent) ||
      misaligned(logits) || misaligned(workspace))
    return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  return run_latent_router(plan, x, w_latent, w_router, latent, logits, nullptr, nullptr, workspace,
                           rows, false, static_cast<hipStream_t>(stream));
}

int route_topk16(const route_plan* plan, const float* logits, int32_t* ids, float* weights,
                 int32_t rows, void* stream) {
  if (!plan || !logits || !ids || !weights) return ROUTE_E_ARG;
  if (is_share(plan)) return ROUTE_E_SHAPE;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(logits) || misaligned(ids) || misaligned(weights)) return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  return status_of(route::launch_topk16(logits, ids, weights, rows, static_cast<hipStream_t>(stream)));
}

int route_fused(const route_plan* plan, const void* x, const void* w_latent, const float* w_router,
                void* latent, float* logits, int32_t* ids, float* weights, void* workspace,
                int32_t rows, void* stream) {
  if (!plan || !x || !w_latent || !w_router || !latent || !ids || !weights || !workspace)
    return ROUTE_E_ARG;
  if (is_share(plan)) return ROUTE_E_SHAPE;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(x) || misaligned(w_latent) || misaligned(w_router) || misaligned(latent) ||
      (logits && misaligned(logits)) || misaligned(ids) || misaligned(weights) || misaligned(workspace))
    return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  float* lg = logits ? logits
                     : reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->off_logits);
  return run_latent_router(plan, x, w_latent, w_router, latent, lg, ids, weights, workspace, rows,
                           true, static_cast<hipStream_t>(stream));
}

int route_topk16_sharded(const route_plan* plan, const float* logits, int32_t shards, int32_t* ids,
                         float* weights, void* workspace, int32_t rows, void* stream) {
  if (!plan || !logits || !ids || !weights || !workspace) return ROUTE_E_ARG;
  if (!route::topk16_shards_valid(shards)) return ROUTE_E_ARG;
  if (is_share(plan)) return ROUTE_E_SHAPE;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(logits) || misaligned(ids) || misaligned(weights) || misaligned(workspace))
    return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  uint64_t* cand = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + plan->off_cand);
  return status_of(route::launch_topk16_sharded(logits, shards, ids, weights, cand, rows,
                                                static_cast<hipStream_t>(stream)));
}

size_t route_packed_weight_bytes(const route_plan* plan) {
  return plan && packed_plan(plan) ? packed_bytes(plan) : 0;
}

int route_pack_weights(const route_plan* plan, const void* w_latent, const float* w_router,
                       void* packed, void* stream) {
  if (!plan || !w_latent || !w_router || !packed) return ROUTE_E_ARG;
  if (!packed_plan(plan)) return ROUTE_E_SHAPE;
  if (misaligned(w_latent) || misaligned(w_router) || misaligned(packed)) return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  const uint16_t* wl = static_cast<const uint16_t*>(w_latent);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(plan->mode == ROUTE_MODE_DECODE ? route::launch_pack_decode_weights(wl, w_router, packed, s)
                                                   : route::launch_pack_prefill_weights(wl, w_router, packed, s));
}

int route_latent_router_packed(const route_plan* plan, const void* x, const void* packed,
                               void* latent, float* logits, void* workspace, int32_t rows,
                               void* stream) {
  if (!plan || !x || !packed || !latent || !logits || !workspace) return ROUTE_E_ARG;
  if (!packed_plan(plan)) return ROUTE_E_SHAPE;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(x) || misaligned(packed) || misaligned(latent) || misaligned(logits) ||
      misaligned(workspace))
    return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  return run_latent_router(plan, x, packed, packed_router(plan, packed), latent, logits, nullptr, nullptr,
                           workspace, rows, false, static_cast<hipStream_t>(stream), true);
}

int route_fused_packed(const route_plan* plan, const void* x, const void* packed, void* latent,
                       float* logits, int32_t* ids, float* weights, void* workspace, int32_t rows,
                       void* stream) {
  if (!plan || !x || !packed || !latent || !ids || !weights || !workspace) return ROUTE_E_ARG;
  if (!packed_plan(plan)) return ROUTE_E_SHAPE;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(x) || misaligned(packed) || misaligned(latent) || (logits && misaligned(logits)) ||
      misaligned(ids) || misaligned(weights) || misaligned(workspace))
    return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  float* lg = logits ? logits
                     : reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->off_logits);
  return run_latent_router(plan, x, packed, packed_router(plan, packed), latent, lg, ids, weights, workspace,
                           rows, true, static_cast<hipStream_t>(stream), true);
}

int route_fused_packed_noalloc(const route_plan* plan, const void* x, const void* packed, void* latent,
                               float* logits, int32_t* ids, float* weights, int32_t rows, void* stream) {
  if (!plan || !x || !packed || !latent || !ids || !weights) return ROUTE_E_ARG;
  if (!packed_plan(plan)) return ROUTE_E_SHAPE;
  if (int st = check_rows(plan, rows)) return st;
  if (misaligned(x) || misaligned(packed) || misaligned(latent) || (logits && misaligned(logits)) ||
      misaligned(ids) || misaligned(weights))
    return ROUTE_E_ALIGN;
  if (int st = check_device(plan)) return st;
  size_t cap = 0;
  void* scratch = route::static_scratch(plan->device, &cap);
  if (scratch == nullptr) return ROUTE_E_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan->mode == ROUTE_MODE_DECODE) {
    float* lg_buf = nullptr;
    const route::DecodeWorkspace ws = route::static_decode_workspace(scratch, &lg_buf);
    // the static partial areas are laid out for ROUTE_DECODE_MAX_ROWS rows
    return status_of(route::launch_decode_route(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(packed), packed_router(plan, packed),
        static_cast<uint16_t*>(latent), logits ? logits : lg_buf, ids, weights, ws, rows,
        ROUTE_DECODE_MAX_ROWS, plan->latent, plan->experts, true, true, s));
  }
  // prefill: the scratch holds the logits only when the caller passes none,
  // past the decode counters
  float* lg = logits;
  if (lg == nullptr) {
    const size_t off = route::static_free_offset();
    if ((size_t)rows * ROUTE_EXPERTS * sizeof(float) > cap - off) return ROUTE_E_SCRATCH;
    lg = reinterpret_cast<float*>(static_cast<char*>(scratch) + off);
  }
  // (no workspace for K-split partials: the GEMMs run unsplit)
  return run_prefill_packed(x, packed, latent, lg, ids, weights, rows, true, nullptr, s);
}

void route_destroy(route_plan* plan) { delete plan; }

const char* route_strerror(int status) {
  switch (status) {
    case ROUTE_OK: return "ok";
    case ROUTE_E_ARG: return "invalid argument (NULL pointer, ABI version or mode)";
    case ROUTE_E_ROWS: return "row count outside the prepared envelope";
    case ROUTE_E_SHAPE:
      return "shape is not hidden 7168 / top-16 with latent x experts 3584 x 896 (or, decode only, "
             "a rank share 448 x 112 or 224 x 56), or the call needs the whole route";
    case ROUTE_E_ALIGN: return "device pointer not 16-byte aligned";
    case ROUTE_E_DEVICE: return "device missing, not gfx950, or not the current device";
    case ROUTE_E_HIP: return "HIP launch failed";
    case ROUTE_E_SCRATCH:
      return "the call needs more device scratch than the library's static scratch holds (pass "
             "logits, or call route_fused_packed with a workspace)";
    default: return "unknown status";
  }
}

}  // extern "C"
