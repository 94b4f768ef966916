/*
 * route.h - C ABI of the per-row MoE route on one AMD Instinct MI355X (gfx950).
 *
 * For each token row the route computes
 *   latent[r, n] = BF16( sum_{k<7168} x[r, k] * W[k, n] ),  n < 3584
 *       one full-K dot product per output, accumulated in FP32 (partials of
 *       the K split combined in FP64) and rounded to BF16 once, nearest-even;
 *       page "Optionally gather the Kimi3 prefill latent instead of reducing
 *       it" (voipmonitor/flare pull request 16), Description, numerics bullet;
 *   logits[r, e] = FP32( sum_k x[r, k] * Wr[k, e] ),  e < 896
 *       FP32 router logits, accumulated in FP64 at decode and in FP32 runs
 *       folded into FP64 at prefill, rounded once; page "Use two row blocks
 *       for eight-row Kimi paired gathers" (NVIDIA/hyperflare-inference pull
 *       request 265) gives the router output as FP32;
 *   ids[r, 0..15], weights[r, 0..15]
 *       the standalone top-16: the 16 experts with the largest logits, ordered
 *       by (logit descending, expert index ascending), -0.0 equal to +0.0, NaN
 *       below -inf; weights are sigmoid(logit) normalised to sum 1 over the
 *       16, computed in FP64 and rounded to FP32; page "Kimi K3.1 recipe:
 *       route 9..20 decode rows through the pushed pair gather and standalone
 *       top-16" (voipmonitor/flare pull request 24), "What / why" and
 *       "Dependency".
 *
 * Envelope: a plan is prepared once for a mode, a row capacity and an output
 * shape (the whole route, or a rank share below); decode
 * plans accept 1..20 rows (the same page, "What / why": rounds of 1..20 rows
 * are prepared, anything else raises at preparation), prefill plans 1..3072
 * rows (the 3072-row chunk of pull request 16's timing table). There is no
 * fallback: every error is a negative status, and an argument error launches
 * nothing.
 *
 * Ownership and threading:
 *   - the caller owns every device buffer (inputs, weights, outputs,
 *     workspace); the library allocates no device memory and never
 *     synchronises; run calls only enqueue kernels on `stream`, so they can be
 *     captured into a HIP graph;
 *   - the workspace (route_workspace_bytes) must be zero-filled once by the
 *     caller before its first use; decode calls keep a few counters in it
 *     from one call to the next, so it must not be modified between calls
 *     (zero-filling it again is allowed). Two calls that overlap in time must
 *     use different workspaces;
 *   - a plan is immutable after route_prepare and may be shared by threads.
 *
 * Layouts (row-major, all device pointers, 16-byte aligned):
 *   x        [rows][7168]   BF16 (uint16 bit patterns)
 *   w_latent [7168][3584]   BF16   ([K][N], N contiguous)
 *   w_router [7168][896]    FP32   ([K][E], E contiguous)
 *   latent   [rows][3584]   BF16
 *   logits   [rows][896]    FP32
 *   ids      [rows][16]     int32, selection order
 *   weights  [rows][16]     FP32, same order as ids
 *
 * Rank shares (decode only): a decode plan may instead be prepared for one
 * tensor-parallel rank's share of the route, latent x experts = 448 x 112 (8
 * ranks) or 224 x 56 (16 ranks): the per-rank output shapes of page "Use two
 * row blocks for eight-row Kimi paired gathers" (BF16 [8, 224] latent and FP32
 * [8, 56] router at 16 ranks) and of page "Optionally gather the Kimi3 prefill
 * latent instead of reducing it" (448 latent columns per rank at 8 ranks).
 * Every 3584 and 896 above then reads as the share's latent and experts:
 * w_latent [7168][latent] and w_router [7168][experts] are the rank's
 * contiguous column slices of the full weights (copied out by the caller),
 * and latent/logits have that many columns. Each output is still one full-K
 * dot product rounded once, within the same bounds as the whole route's (the
 * K split differs, so the last bit may differ from the whole route's
 * corresponding column). A share has no top-16 (its experts are a fraction
 * of the route's): route_topk16, route_fused and route_topk16_sharded return
 * ROUTE_E_SHAPE on a share plan.
 *
 * `stream` is a hipStream_t (NULL = the null stream); the current HIP device
 * must be the plan's device.
 */
#ifndef ROUTE_H
#define ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROUTE_ABI_VERSION 1u
#define ROUTE_HIDDEN 7168
#define ROUTE_LATENT 3584
#define ROUTE_EXPERTS 896
#define ROUTE_TOPK 16
#define ROUTE_DECODE_MAX_ROWS 20
#define ROUTE_PREFILL_MAX_ROWS 3072

/* Status codes. 0 is success; every error is negative. Every argument error
 * is found before anything is launched. */
#define ROUTE_OK 0
#define ROUTE_E_ARG (-1)    /* NULL pointer, bad abi_version or unknown mode */
#define ROUTE_E_ROWS (-2)   /* rows outside the mode's envelope, or above the plan's */
#define ROUTE_E_SHAPE (-3)  /* hidden/topk not 7168/16, latent x experts not 3584 x 896
                               (or a decode share 448 x 112 / 224 x 56), or a
                               top-16 call on a share plan */
#define ROUTE_E_ALIGN (-4)  /* a device pointer is not 16-byte aligned */
#define ROUTE_E_DEVICE (-5) /* no such device, not gfx950, or not the current device */
#define ROUTE_E_HIP (-6)    /* the HIP runtime rejected one of the call's launches (the
                               launch's own status, not an error left by earlier
                               calls); kernels of the call enqueued before it
                               stay enqueued */
#define ROUTE_E_SCRATCH (-7) /* route_fused_packed_noalloc: the call needs more than
                                the library's static scratch holds */

typedef enum { ROUTE_MODE_DECODE = 0, ROUTE_MODE_PREFILL = 1 } route_mode;

typedef struct {
  uint32_t abi_version; /* ROUTE_ABI_VERSION */
  int32_t mode;         /* route_mode */
  int32_t rows;         /* the most rows any call on this plan passes */
  int32_t hidden;       /* 7168 */
  int32_t latent;       /* 3584; decode shares: 448 or 224 */
  int32_t experts;      /* 896; decode shares: 112 or 56 (with 448 / 224) */
  int32_t topk;         /* 16 */
  int32_t device;       /* HIP device ordinal */
} route_config;

typedef struct route_plan route_plan; /* opaque, host memory, immutable */

/* Validate cfg and build a plan. Arguments are checked in this order before
 * any HIP call: cfg/out non-NULL and abi_version (ROUTE_E_ARG), mode
 * (ROUTE_E_ARG), shape fields (ROUTE_E_SHAPE), rows (ROUTE_E_ROWS); then the
 * device must exist and be gfx950 (ROUTE_E_DEVICE). On error *out is NULL. */
int route_prepare(const route_config* cfg, route_plan** out);

/* Bytes of device workspace the plan's run calls need (a multiple of 256;
 * 0 for a NULL plan). Zero-fill it once before first use. */
size_t route_workspace_bytes(const route_plan* plan);

/* Latent projection and router logits for `rows` rows (1..plan rows).
 * Every pointer is required. Prefill plans run the router on three exact BF16
 * parts of each FP32 weight, then recompute every logit that came out as an
 * infinity or a NaN (a hidden row holding an infinity or a NaN, or an FP32
 * partial sum that overflowed) as an exact FP64 dot, so such rows get the
 * plain dot's IEEE result. Prefill calls of at most 1,728 rows split K over
 * more workgroups (their partial sums go through the workspace and are added
 * in FP64 before the single rounding), so a row's last bit may depend on the
 * call's row count; calls of more rows do not split. */
int route_latent_router(const route_plan* plan, const void* x, const void* w_latent,
                        const float* w_router, void* latent, float* logits,
                        void* workspace, int32_t rows, void* stream);

/* Standalone top-16 of `rows` rows of FP32 logits (1..plan rows). A share
 * plan returns ROUTE_E_SHAPE. */
int route_topk16(const route_plan* plan, const float* logits, int32_t* ids,
                 float* weights, int32_t rows, void* stream);

/* The whole route in one call; bitwise equal to route_latent_router followed by
 * route_topk16 on the same plan. `logits` may be NULL (the logits then live in
 * the workspace). Decode plans select inside the projection kernel (one
 * launch); prefill plans launch the top-16 after the two GEMMs. */
int route_fused(const route_plan* plan, const void* x, const void* w_latent,
                const float* w_router, void* latent, float* logits, int32_t* ids,
                float* weights, void* workspace, int32_t rows, void* stream);

/* Sharded top-16: the selection half of a route whose 896 experts are split
 * into `shards` contiguous shards of 896 / shards experts (shards in {1, 2, 4,
 * 7, 8, 14, 16, 28, 32, 56}: a divisor of 896 with at least 16 experts per
 * shard; 8 and 16 are the tensor-parallel widths of page "Use two row blocks
 * for eight-row Kimi paired gathers", whose per-rank router output is 56
 * experts). Stage 1 selects each shard's local top-16 into the workspace,
 * stage 2 merges the 16 * shards candidates into the global top-16 and its
 * weights. The merge is exact: the output is bitwise that of route_topk16 on
 * the same logits. Any other `shards` is ROUTE_E_ARG; `workspace` is the
 * plan's workspace (its candidate area is used; no counters). */
int route_topk16_sharded(const route_plan* plan, const float* logits, int32_t shards, int32_t* ids,
                         float* weights, void* workspace, int32_t rows, void* stream);

/* Packed weights. Weights are model parameters, loaded once; each kernel
 * reads them fastest in an order of its own, so route_pack_weights reorders
 * both weights once into the plan's packed format, and the *_packed calls
 * then read that buffer in place of w_latent and w_router. Every output
 * keeps the definitions and bounds above.
 *   decode (whole route): both weights in the decode kernel's consumption
 *     order, so every workgroup streams one contiguous block with 16-byte
 *     loads (the [K][N] layouts give it strided 128-byte row segments);
 *     77,070,336 bytes: the latent weight's 51,380,224 bytes of BF16 values,
 *     then the router weight's 25,690,112 bytes of FP32 values, each tile in
 *     K order. The kernel splits K its own ways (8 for both weights up to 4
 *     rows, 4 for the latent and 8 for the router above); this K split
 *     differs from the [K][N] kernel's, so a latent value may differ from
 *     route_fused's in the last bit (each is one full-K dot rounded once),
 *     and between a packed call of 1..4 rows and one of 5..20 rows. The
 *     [K][N] kernel splits the latent 4 ways at every width, so its latent
 *     for a row does not depend on the call's row count. Logits are FP64
 *     sums rounded once in both;
 *   prefill: the weights K-contiguous, W as [3584][7168] BF16 (the [out][in]
 *     layout of a linear layer) and the router weight as its three exact
 *     BF16 parts [2688][7168] (split once here instead of on every call), so
 *     the GEMMs read both operands with 16-byte LDS reads; 89,915,392 bytes.
 *     Every GEMM lane receives the same operand values in the same order as
 *     with [K][N] weights: the results are bitwise those of route_fused.
 *     (The split is exact for router weights below 2^128 * (1 - 2^-9) in
 *     magnitude, the largest BF16 value.)
 * Share plans have no packed format: route_packed_weight_bytes returns 0 and
 * the packed calls return ROUTE_E_SHAPE. */

/* Bytes of the plan's packed buffer (decode 77,070,336, prefill 89,915,392),
 * or 0 for a NULL or share plan. */
size_t route_packed_weight_bytes(const route_plan* plan);

/* Write the packed buffer `packed` (caller-owned, route_packed_weight_bytes
 * bytes, 16-byte aligned) from w_latent [7168][3584] BF16 and w_router
 * [7168][896] FP32; enqueued on `stream`. Every pointer is required; the
 * buffer must not overlap the weights. A decode buffer serves decode plans
 * and a prefill buffer prefill plans, of any row capacity. */
int route_pack_weights(const route_plan* plan, const void* w_latent, const float* w_router,
                       void* packed, void* stream);

/* route_latent_router with packed weights. */
int route_latent_router_packed(const route_plan* plan, const void* x, const void* packed,
                               void* latent, float* logits, void* workspace, int32_t rows,
                               void* stream);

/* route_fused with packed weights (`logits` may be NULL). */
int route_fused_packed(const route_plan* plan, const void* x, const void* packed, void* latent,
                       float* logits, int32_t* ids, float* weights, void* workspace, int32_t rows,
                       void* stream);

/* route_fused_packed without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). It allocates nothing and calls no allocating
 * routine: its scratch is a static device array inside the library, one per
 * GPU, ROUTE_STATIC_SCRATCH_BYTES bytes, held until the process ends; its
 * address is taken and the array cleared when the first plan for the device
 * is prepared. Decode plans (whole route, 1..20 rows) keep their counters and
 * split-K partials there, and their logits when `logits` is NULL; prefill
 * plans use it only for the logits when `logits` is NULL, at most
 * ROUTE_STATIC_SCRATCH_BYTES - 512 bytes (rows * 3584 bytes), and return
 * ROUTE_E_SCRATCH above that. Outputs are bitwise those of route_fused_packed
 * on the same plan, except prefill calls of at most 1,728 rows: there
 * route_fused_packed splits K with partials in its workspace and this call
 * does not (the static scratch cannot hold them), so a value may differ in
 * the last bit, both within the same bounds, and such a call takes about as
 * long as a 3072-row chunk. Every call on a GPU shares that GPU's array, and
 * the decode counters carry over from call to call: two calls that overlap
 * in time on one GPU (different streams, threads or graphs running at once)
 * race on it and must not be issued. Other statuses as route_fused_packed;
 * ROUTE_E_HIP if the array's address could not be taken for the device. */
#define ROUTE_STATIC_SCRATCH_BYTES 3512832u
int route_fused_packed_noalloc(const route_plan* plan, const void* x, const void* packed, void* latent,
                               float* logits, int32_t* ids, float* weights, int32_t rows,
                               void* stream);

/* Free a plan (NULL is accepted). */
void route_destroy(route_plan* plan);

/* Static description of a status code. */
const char* route_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ROUTE_H */
