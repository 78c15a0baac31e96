/* A plain C client of libloki.so: no Python, no torch, only the C ABI of
 * include/loki.h and the HIP runtime for device memory.  It calibrates a
 * basis on the host, appends a synthetic cache, decodes on every path and
 * checks what holds without an oracle: ascending in-range ids, identical
 * selections and near-identical outputs on every path, decode with k = S
 * equal to the dense baseline, and the argument checks.  Prints "ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "loki.h"

#define FAIL(...)                     \
  do {                                \
    fprintf(stderr, "FAIL: ");        \
    fprintf(stderr, __VA_ARGS__);     \
    fprintf(stderr, "\n");            \
    return 1;                         \
  } while (0)
#define HIPOK(x)                                                   \
  do {                                                             \
    hipError_t e_ = (x);                                           \
    if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_)); \
  } while (0)
#define LOKIOK(x)                                                   \
  do {                                                              \
    int s_ = (x);                                                   \
    if (s_ != LOKI_OK) FAIL("%s: %s", #x, loki_status_string(s_));  \
  } while (0)

enum { B = 2, HQ = 4, HKV = 2, D = 64, DS = 16, S = 300, SMAX = 320, K = 75, NCAL = 512 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, 53 random bits */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
static double gauss(void) {
  double u = uniform(), v = uniform();
  if (u < 1e-300) u = 1e-300;
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
/* keys with a decaying spectrum along the coordinate axes */
static float key_elem(int i) { return (float)(gauss() * exp(-(double)i / 8.0)); }

static int decode(int path, int k, const float* q, const float* slab, const float* rest,
                  const float* v, const float* P, float* out, int32_t* idx, void* ws, size_t wsb) {
  return loki_decode_ex(q, slab, rest, v, P, B, HQ, HKV, D, DS, S, SMAX, k, LOKI_F32, out, idx, ws,
                        wsb, path, NULL);
}

int main(void) {
  if (loki_abi_version() != LOKI_ABI_VERSION) FAIL("ABI %d, header %d", loki_abi_version(), LOKI_ABI_VERSION);

  /* host data */
  static float cal[NCAL * D], P[HKV * D * D], kh[B * HKV * S * D], vh[B * HKV * S * D], qh[B * HQ * D];
  for (int g = 0; g < HKV; ++g) {
    for (int n = 0; n < NCAL * D; ++n) cal[n] = key_elem(n % D);
    LOKIOK(loki_calibrate(cal, NCAL, D, P + g * D * D, NULL));
  }
  for (int n = 0; n < B * HKV * S * D; ++n) {
    kh[n] = key_elem(n % D);
    vh[n] = (float)gauss();
  }
  for (int n = 0; n < B * HQ * D; ++n) qh[n] = (float)gauss();

  /* device buffers: the caller owns them all */
  float *dk, *dv, *dq, *dP, *slab, *rest, *vc, *out, *out2;
  int32_t *idx, *idx2;
  void* ws;
  const size_t wsb = loki_decode_workspace_size(B, HQ, SMAX, D, S);
  if (wsb == 0 || wsb % 256) FAIL("workspace size %zu", wsb);
  HIPOK(hipMalloc((void**)&dk, sizeof kh));
  HIPOK(hipMalloc((void**)&dv, sizeof vh));
  HIPOK(hipMalloc((void**)&dq, sizeof qh));
  HIPOK(hipMalloc((void**)&dP, sizeof P));
  HIPOK(hipMalloc((void**)&slab, (size_t)B * HKV * SMAX * DS * 4));
  HIPOK(hipMalloc((void**)&rest, (size_t)B * HKV * SMAX * (D - DS) * 4));
  HIPOK(hipMalloc((void**)&vc, (size_t)B * HKV * SMAX * D * 4));
  HIPOK(hipMalloc((void**)&out, (size_t)B * HQ * D * 4));
  HIPOK(hipMalloc((void**)&out2, (size_t)B * HQ * D * 4));
  HIPOK(hipMalloc((void**)&idx, (size_t)B * HQ * S * 4));
  HIPOK(hipMalloc((void**)&idx2, (size_t)B * HQ * S * 4));
  HIPOK(hipMalloc(&ws, wsb));
  HIPOK(hipMemcpy(dk, kh, sizeof kh, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(dv, vh, sizeof vh, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(dq, qh, sizeof qh, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(dP, P, sizeof P, hipMemcpyHostToDevice));

  /* append all S tokens at position 0 (null stream) */
  LOKIOK(loki_kv_append(dk, dv, dP, slab, rest, vc, B, HKV, D, DS, SMAX, 0, S, LOKI_F32, NULL));

  /* every path: ids ascending and in range, the same selection, outputs close */
  static int32_t ih[4][B * HQ * K];
  static float oh[4][B * HQ * D];
  const int paths[4] = {LOKI_PATH_AUTO, LOKI_PATH_FUSED, LOKI_PATH_SPLIT, LOKI_PATH_UNION};
  for (int p = 0; p < 4; ++p) {
    LOKIOK(decode(paths[p], K, dq, slab, rest, vc, dP, out, idx, ws, wsb));
    HIPOK(hipDeviceSynchronize());
    HIPOK(hipMemcpy(ih[p], idx, sizeof ih[p], hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(oh[p], out, sizeof oh[p], hipMemcpyDeviceToHost));
    for (int r = 0; r < B * HQ; ++r)
      for (int t = 0; t < K; ++t) {
        const int32_t j = ih[p][r * K + t];
        if (j < 0 || j >= S || (t > 0 && j <= ih[p][r * K + t - 1])) FAIL("path %d row %d: bad id %d", paths[p], r, j);
      }
    if (memcmp(ih[p], ih[0], sizeof ih[p]) != 0) FAIL("path %d selects differently", paths[p]);
    for (int n = 0; n < B * HQ * D; ++n)
      if (!(fabsf(oh[p][n] - oh[0][n]) <= 1e-5f)) FAIL("path %d output %d differs", paths[p], n);
  }

  /* k = S keeps every token: the same function as the dense baseline */
  static float full[B * HQ * D], dense[B * HQ * D];
  LOKIOK(decode(LOKI_PATH_SPLIT, S, dq, slab, rest, vc, dP, out, idx2, ws, wsb));
  LOKIOK(loki_dense_decode(dq, slab, rest, vc, dP, B, HQ, HKV, D, DS, S, SMAX, LOKI_F32, out2, ws, wsb, NULL));
  HIPOK(hipDeviceSynchronize());
  HIPOK(hipMemcpy(full, out, sizeof full, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(dense, out2, sizeof dense, hipMemcpyDeviceToHost));
  for (int n = 0; n < B * HQ * D; ++n)
    if (!(fabsf(full[n] - dense[n]) <= 1e-5f)) FAIL("k = S differs from dense at %d: %g vs %g", n, full[n], dense[n]);

  /* argument checks: host-side errors, nothing launched */
  if (decode(LOKI_PATH_SPLIT, 0, dq, slab, rest, vc, dP, out, idx, ws, wsb) != LOKI_EINVAL) FAIL("k = 0 accepted");
  if (decode(LOKI_PATH_SPLIT, K, dq, slab, rest, vc, dP, out, idx, ws, 64) != LOKI_EWORKSPACE) FAIL("small workspace accepted");
  if (loki_decode_path(B, HQ, HKV, D, 18, S, K, LOKI_F32, LOKI_PATH_AUTO) != LOKI_EUNSUPPORTED) FAIL("d*4 not a multiple of 16 accepted");
  if (!loki_status_string(12345)) FAIL("status string");

  hipFree(dk); hipFree(dv); hipFree(dq); hipFree(dP); hipFree(slab); hipFree(rest); hipFree(vc);
  hipFree(out); hipFree(out2); hipFree(idx); hipFree(idx2); hipFree(ws);
  printf("ok\n");
  return 0;
}
