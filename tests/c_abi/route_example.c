/* The route driven from plain C (C99) through include/route.h and the HIP
 * runtime API, the way a C or C++ serving loop would use it: prepare a plan,
 * allocate and zero the workspace once, run route_fused on an 8-row decode
 * batch, and run route_latent_router + route_topk16 on the same inputs.
 *
 * Checks (properties that hold for any inputs; value parity against the
 * oracle lives in the Python tests):
 *   - the fused call equals the two calls bit for bit;
 *   - per row, the ids are 16 distinct experts in selection order: logits
 *     non-increasing, lower index first among equal logits, and no other
 *     expert above the 16th (or equal to it with a lower index);
 *   - the weights are positive and sum to 1 within 1e-5;
 *   - a few latent values agree with a double-precision dot on the host
 *     within one BF16 ULP (plus 2^-20 of the sum of the terms' magnitudes,
 *     the FP32 accumulation band);
 *   - a call with more rows than the plan returns ROUTE_E_ROWS and writes
 *     nothing.
 * Exit status 0 and "c example ok" on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "route.h"

#define ROWS 8
#define K ROUTE_HIDDEN
#define N ROUTE_LATENT
#define E ROUTE_EXPERTS

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));              \
      return 1;                                                           \
    }                                                                     \
  } while (0)

static uint64_t lcg_state = 0x2545F4914F6CDD1Dull;

/* uniform in [-1, 1) from a 64-bit linear congruential generator */
static double next_uniform(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg_state >> 11) * (1.0 / 4503599627370496.0) - 1.0;
}

/* float -> BF16 bits, nearest-even (finite inputs) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static int check_selection(const float* lg, const int32_t* ids, const float* w, int r) {
  int seen[E];
  int k, e;
  double sum = 0.0;
  memset(seen, 0, sizeof seen);
  for (k = 0; k < ROUTE_TOPK; ++k) {
    const int id = ids[k];
    if (id < 0 || id >= E || seen[id]) {
      printf("FAIL row %d: id %d at %d out of range or repeated\n", r, id, k);
      return 1;
    }
    seen[id] = 1;
    if (k > 0) {
      const float a = lg[ids[k - 1]], b = lg[id];
      if (a < b || (a == b && ids[k - 1] > id)) {
        printf("FAIL row %d: selection order broken at %d\n", r, k);
        return 1;
      }
    }
    if (!(w[k] > 0.0f)) {
      printf("FAIL row %d: weight %d is %g\n", r, k, (double)w[k]);
      return 1;
    }
    sum += w[k];
  }
  if (fabs(sum - 1.0) > 1e-5) {
    printf("FAIL row %d: weights sum to %.9f\n", r, sum);
    return 1;
  }
  {
    const float last = lg[ids[ROUTE_TOPK - 1]];
    for (e = 0; e < E; ++e) {
      if (seen[e]) continue;
      if (lg[e] > last || (lg[e] == last && e < ids[ROUTE_TOPK - 1])) {
        printf("FAIL row %d: expert %d belongs in the top 16\n", r, e);
        return 1;
      }
    }
  }
  return 0;
}

int main(void) {
  const size_t nx = (size_t)ROWS * K, nw = (size_t)K * N, nwr = (size_t)K * E;
  uint16_t *hx, *hw, *hlat, *hlat2;
  float *hwr, *hlg, *hlg2, *hwt, *hwt2;
  int32_t *hids, *hids2;
  void *dx, *dw, *dwr, *dlat, *dlg, *dids, *dwt, *dlat2, *dlg2, *dids2, *dwt2, *dws;
  route_plan* plan = NULL;
  route_config cfg;
  size_t ws_bytes, i;
  int count = 0, r, n, st, fails = 0;

  HIP_OK(hipGetDeviceCount(&count));
  if (count < 1) {
    printf("FAIL no HIP device\n");
    return 1;
  }
  HIP_OK(hipSetDevice(0));

  memset(&cfg, 0, sizeof cfg);
  cfg.abi_version = ROUTE_ABI_VERSION;
  cfg.mode = ROUTE_MODE_DECODE;
  cfg.rows = ROWS;
  cfg.hidden = K;
  cfg.latent = N;
  cfg.experts = E;
  cfg.topk = ROUTE_TOPK;
  cfg.device = 0;
  st = route_prepare(&cfg, &plan);
  if (st != ROUTE_OK) {
    printf("FAIL route_prepare: %s\n", route_strerror(st));
    return 1;
  }
  ws_bytes = route_workspace_bytes(plan);

  hx = malloc(nx * 2);
  hw = malloc(nw * 2);
  hwr = malloc(nwr * 4);
  hlat = malloc((size_t)ROWS * N * 2);
  hlat2 = malloc((size_t)ROWS * N * 2);
  hlg = malloc((size_t)ROWS * E * 4);
  hlg2 = malloc((size_t)ROWS * E * 4);
  hids = malloc((size_t)ROWS * ROUTE_TOPK * 4);
  hids2 = malloc((size_t)ROWS * ROUTE_TOPK * 4);
  hwt = malloc((size_t)ROWS * ROUTE_TOPK * 4);
  hwt2 = malloc((size_t)ROWS * ROUTE_TOPK * 4);
  if (!hx || !hw || !hwr || !hlat || !hlat2 || !hlg || !hlg2 || !hids || !hids2 || !hwt || !hwt2) {
    printf("FAIL host allocation\n");
    return 1;
  }
  /* hidden ~ U(-1.7, 1.7) (variance about 1), weights scaled by 1/sqrt(K) */
  for (i = 0; i < nx; ++i) hx[i] = to_bf16((float)(1.7320508 * next_uniform()));
  for (i = 0; i < nw; ++i) hw[i] = to_bf16((float)(1.7320508 / 84.664042 * next_uniform()));
  for (i = 0; i < nwr; ++i) hwr[i] = (float)(1.7320508 / 84.664042 * next_uniform());

  HIP_OK(hipMalloc(&dx, nx * 2));
  HIP_OK(hipMalloc(&dw, nw * 2));
  HIP_OK(hipMalloc(&dwr, nwr * 4));
  HIP_OK(hipMalloc(&dlat, (size_t)ROWS * N * 2));
  HIP_OK(hipMalloc(&dlg, (size_t)ROWS * E * 4));
  HIP_OK(hipMalloc(&dids, (size_t)ROWS * ROUTE_TOPK * 4));
  HIP_OK(hipMalloc(&dwt, (size_t)ROWS * ROUTE_TOPK * 4));
  HIP_OK(hipMalloc(&dlat2, (size_t)ROWS * N * 2));
  HIP_OK(hipMalloc(&dlg2, (size_t)ROWS * E * 4));
  HIP_OK(hipMalloc(&dids2, (size_t)ROWS * ROUTE_TOPK * 4));
  HIP_OK(hipMalloc(&dwt2, (size_t)ROWS * ROUTE_TOPK * 4));
  HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMemcpy(dx, hx, nx * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, hw, nw * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dwr, hwr, nwr * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(dws, 0, ws_bytes));
  HIP_OK(hipMemset(dids2, 0xFF, (size_t)ROWS * ROUTE_TOPK * 4));

  /* more rows than the plan: rejected, nothing launched */
  st = route_fused(plan, dx, dw, (const float*)dwr, dlat2, (float*)dlg2, (int32_t*)dids2,
                   (float*)dwt2, dws, ROWS + 1, NULL);
  if (st != ROUTE_E_ROWS) {
    printf("FAIL rows above the plan: status %d\n", st);
    ++fails;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hids2, dids2, (size_t)ROWS * ROUTE_TOPK * 4, hipMemcpyDeviceToHost));
  for (i = 0; i < (size_t)ROWS * ROUTE_TOPK; ++i)
    if (hids2[i] != -1) {
      printf("FAIL a rejected call wrote ids\n");
      ++fails;
      break;
    }

  st = route_fused(plan, dx, dw, (const float*)dwr, dlat, (float*)dlg, (int32_t*)dids, (float*)dwt, dws,
                   ROWS, NULL);
  if (st != ROUTE_OK) {
    printf("FAIL route_fused: %s\n", route_strerror(st));
    return 1;
  }
  st = route_latent_router(plan, dx, dw, (const float*)dwr, dlat2, (float*)dlg2, dws, ROWS, NULL);
  if (st == ROUTE_OK) st = route_topk16(plan, (const float*)dlg2, (int32_t*)dids2, (float*)dwt2, ROWS, NULL);
  if (st != ROUTE_OK) {
    printf("FAIL two-call route: %s\n", route_strerror(st));
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hlat, dlat, (size_t)ROWS * N * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlg, dlg, (size_t)ROWS * E * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hids, dids, (size_t)ROWS * ROUTE_TOPK * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hwt, dwt, (size_t)ROWS * ROUTE_TOPK * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlat2, dlat2, (size_t)ROWS * N * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlg2, dlg2, (size_t)ROWS * E * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hids2, dids2, (size_t)ROWS * ROUTE_TOPK * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hwt2, dwt2, (size_t)ROWS * ROUTE_TOPK * 4, hipMemcpyDeviceToHost));

  if (memcmp(hlat, hlat2, (size_t)ROWS * N * 2) || memcmp(hlg, hlg2, (size_t)ROWS * E * 4) ||
      memcmp(hids, hids2, (size_t)ROWS * ROUTE_TOPK * 4) || memcmp(hwt, hwt2, (size_t)ROWS * ROUTE_TOPK * 4)) {
    printf("FAIL route_fused differs from route_latent_router + route_topk16\n");
    ++fails;
  }
  for (r = 0; r < ROWS; ++r)
    fails += check_selection(hlg + (size_t)r * E, hids + (size_t)r * ROUTE_TOPK, hwt + (size_t)r * ROUTE_TOPK, r);

  /* a few latent outputs against a double-precision dot: within one BF16 ULP */
  for (n = 0; n < 64; ++n) {
    const int rr = n % ROWS, col = (n * 997) % N;
    double dot = 0.0, terms = 0.0, got, ulp;
    int k;
    for (k = 0; k < K; ++k) {
      const double t = from_bf16(hx[(size_t)rr * K + k]) * from_bf16(hw[(size_t)k * N + col]);
      dot += t;
      terms += fabs(t);
    }
    got = from_bf16(hlat[(size_t)rr * N + col]);
    /* one BF16 ULP of the exact value, plus the FP32 accumulation band */
    ulp = (dot != 0.0 ? ldexp(1.0, ilogb(dot) - 7) : 0.0) + ldexp(terms, -20);
    if (fabs(got - dot) > ulp) {
      printf("FAIL latent[%d][%d] = %.9g, host dot %.9g\n", rr, col, got, dot);
      ++fails;
    }
  }

  hipFree(dx);
  hipFree(dw);
  hipFree(dwr);
  hipFree(dlat);
  hipFree(dlg);
  hipFree(dids);
  hipFree(dwt);
  hipFree(dlat2);
  hipFree(dlg2);
  hipFree(dids2);
  hipFree(dwt2);
  hipFree(dws);
  route_destroy(plan);
  free(hx);
  free(hw);
  free(hwr);
  free(hlat);
  free(hlat2);
  free(hlg);
  free(hlg2);
  free(hids);
  free(hids2);
  free(hwt);
  free(hwt2);
  if (fails == 0) printf("c example ok\n");
  return fails == 0 ? 0 : 1;
}
