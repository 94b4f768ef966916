/* Host-only check of the C ABI from plain C (C99): include/route.h compiles
 * as C, every declared function links against libroute.so, and the calls
 * that validate before touching the HIP runtime return the documented status
 * codes. No GPU is needed: route_prepare checks arguments, shapes and rows
 * before it asks for a device, and the run calls reject a NULL plan first. */
#include <stdio.h>
#include <string.h>

#include "route.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static route_config config(route_mode mode, int32_t rows) {
  route_config c;
  memset(&c, 0, sizeof c);
  c.abi_version = ROUTE_ABI_VERSION;
  c.mode = mode;
  c.rows = rows;
  c.hidden = ROUTE_HIDDEN;
  c.latent = ROUTE_LATENT;
  c.experts = ROUTE_EXPERTS;
  c.topk = ROUTE_TOPK;
  c.device = 0;
  return c;
}

int main(void) {
  route_plan* plan = NULL;
  route_config c;

  expect(route_prepare(NULL, &plan), ROUTE_E_ARG, "NULL config");
  c = config(ROUTE_MODE_DECODE, 8);
  expect(route_prepare(&c, NULL), ROUTE_E_ARG, "NULL out");
  c.abi_version = ROUTE_ABI_VERSION + 1;
  expect(route_prepare(&c, &plan), ROUTE_E_ARG, "abi version");
  c = config((route_mode)7, 8);
  expect(route_prepare(&c, &plan), ROUTE_E_ARG, "unknown mode");
  c = config(ROUTE_MODE_DECODE, ROUTE_DECODE_MAX_ROWS + 1);
  expect(route_prepare(&c, &plan), ROUTE_E_ROWS, "decode rows above the envelope");
  c = config(ROUTE_MODE_DECODE, 0);
  expect(route_prepare(&c, &plan), ROUTE_E_ROWS, "zero rows");
  c = config(ROUTE_MODE_PREFILL, ROUTE_PREFILL_MAX_ROWS + 1);
  expect(route_prepare(&c, &plan), ROUTE_E_ROWS, "prefill rows above the envelope");
  c = config(ROUTE_MODE_DECODE, 8);
  c.hidden = 4096;
  expect(route_prepare(&c, &plan), ROUTE_E_SHAPE, "hidden");
  c = config(ROUTE_MODE_DECODE, 8);
  c.topk = 8;
  expect(route_prepare(&c, &plan), ROUTE_E_SHAPE, "topk");
  c = config(ROUTE_MODE_PREFILL, 64);
  c.latent = 448;
  c.experts = 112;
  expect(route_prepare(&c, &plan), ROUTE_E_SHAPE, "rank share in prefill mode");
  if (plan != NULL) {
    printf("FAIL a rejected prepare wrote a plan\n");
    ++failures;
  }

  expect(route_latent_router(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG,
         "route_latent_router without a plan");
  expect(route_topk16(NULL, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG, "route_topk16 without a plan");
  expect(route_fused(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG,
         "route_fused without a plan");
  expect(route_topk16_sharded(NULL, NULL, 8, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG,
         "route_topk16_sharded without a plan");
  expect(route_pack_weights(NULL, NULL, NULL, NULL, NULL), ROUTE_E_ARG, "route_pack_weights without a plan");
  expect(route_latent_router_packed(NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG,
         "route_latent_router_packed without a plan");
  expect(route_fused_packed(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG,
         "route_fused_packed without a plan");
  expect(route_fused_packed_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL), ROUTE_E_ARG,
         "route_fused_packed_noalloc without a plan");
  if (route_workspace_bytes(NULL) != 0 || route_packed_weight_bytes(NULL) != 0) {
    printf("FAIL sizes of a NULL plan are not 0\n");
    ++failures;
  }
  route_destroy(NULL);

  {
    const int codes[] = {ROUTE_OK, ROUTE_E_ARG, ROUTE_E_ROWS, ROUTE_E_SHAPE,
                         ROUTE_E_ALIGN, ROUTE_E_DEVICE, ROUTE_E_HIP, ROUTE_E_SCRATCH};
    const int n = (int)(sizeof codes / sizeof codes[0]);
    int i, j;
    for (i = 0; i < n; ++i) {
      const char* a = route_strerror(codes[i]);
      if (a == NULL || a[0] == '\0') {
        printf("FAIL route_strerror(%d) is empty\n", codes[i]);
        ++failures;
        continue;
      }
      for (j = 0; j < i; ++j)
        if (strcmp(a, route_strerror(codes[j])) == 0) {
          printf("FAIL route_strerror(%d) repeats route_strerror(%d)\n", codes[i], codes[j]);
          ++failures;
        }
    }
  }

  if (failures == 0) printf("c abi ok\n");
  return failures == 0 ? 0 : 1;
}
