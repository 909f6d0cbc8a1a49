/* The C ABI used from plain C99 (no Python, no C++): host-only calls, and
 * with the argument "gpu" one layer on all-zero weights, whose result has a
 * closed form.  Prints "ok" and returns 0, or names the first failed check
 * and returns 1.
 *
 * All-zero blobs and router ("Flash-MoE: Running a 397B Parameter Model on a
 * Laptop", hysenlabs.com, section "How the SSD expert streaming pipeline
 * works": router -> softmax -> top-K -> experts -> combine): every logit is 0,
 * so the top-K are experts 0 .. K-1 (ties go to the lower index), each with
 * weight 1/K after renormalisation; every dequantised weight is 0 * q + 0, so
 * y is exactly 0. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

#ifdef MOE_C_GPU
#include <hip/hip_runtime_api.h>
#endif

#define CHECK(c, what)                          \
  do {                                          \
    if (!(c)) {                                 \
      printf("failed: %s\n", what);             \
      return 1;                                 \
    }                                           \
  } while (0)

static int host_checks(void) {
  moe_dims d = {4096, 1024, 512, 4, 64, 4, 1};
  size_t off[6];
  CHECK(moe_abi_version() == MOE_ABI_VERSION, "abi version");
  CHECK(moe_check_dims(&d) == MOE_OK, "valid dims");
  CHECK(moe_expert_bytes(&d) == 7077888u, "4-bit blob bytes");
  CHECK(moe_blob_layout(&d, off) == MOE_OK && off[MOE_SEC_GATE_Q] == 0, "blob layout");
  CHECK(moe_workspace_bytes(&d, 1) > 0 && moe_workspace_bytes(&d, 4096) > 0, "workspace bytes");
  CHECK(strcmp(moe_status_str(MOE_ERR_WORKSPACE), "workspace too small") == 0, "status string");
  CHECK(strcmp(moe_status_str(123), "unknown status") == 0, "unknown status");
  d.group = 32;
  CHECK(moe_check_dims(&d) == MOE_ERR_UNSUPPORTED, "group 32 unsupported");
  d.group = 64;
  d.hidden = 3000;
  CHECK(moe_check_dims(&d) == MOE_ERR_SHAPE, "hidden 3000 rejected");
  CHECK(moe_check_dims(NULL) == MOE_ERR_NULL, "null dims");
  return 0;
}

#ifdef MOE_C_GPU
static int gpu_checks(int T) {
  const moe_dims d = {256, 256, 8, 2, 64, 4, 1};
  const size_t blob = moe_expert_bytes(&d), H = 256, K = 2;
  const size_t wsb = moe_workspace_bytes(&d, T);
  void *experts = NULL, *shared = NULL, *router = NULL, *x = NULL, *y = NULL, *ids = NULL,
       *w = NULL, *ws = NULL;
  float yh[4 * 256], wh[4 * 2];
  int32_t idh[4 * 2];
  uint16_t xh[4 * 256];
  size_t i;
  moe_layer L;
  CHECK(T >= 1 && T <= 4, "T");
  CHECK(hipMalloc(&experts, 8 * blob) == hipSuccess && hipMalloc(&shared, blob) == hipSuccess &&
            hipMalloc(&router, 8 * H * 2) == hipSuccess && hipMalloc(&x, T * H * 2) == hipSuccess &&
            hipMalloc(&y, T * H * 4) == hipSuccess && hipMalloc(&ids, T * K * 4) == hipSuccess &&
            hipMalloc(&w, T * K * 4) == hipSuccess && hipMalloc(&ws, wsb) == hipSuccess,
        "hipMalloc");
  CHECK(hipMemset(experts, 0, 8 * blob) == hipSuccess && hipMemset(shared, 0, blob) == hipSuccess &&
            hipMemset(router, 0, 8 * H * 2) == hipSuccess && hipMemset(ws, 0, wsb) == hipSuccess,
        "hipMemset");
  for (i = 0; i < (size_t)T * H; ++i) xh[i] = (uint16_t)(0x3F80u + (i % 7));  /* bf16 ~1 */
  CHECK(hipMemcpy(x, xh, T * H * 2, hipMemcpyHostToDevice) == hipSuccess, "copy x");
  L.router = (const uint16_t *)router;
  L.experts = (const uint8_t *)experts;
  L.expert_stride = (int64_t)blob;
  L.shared = (const uint8_t *)shared;
  /* a zero-filled workspace needs no moe_workspace_init */
  CHECK(moe_layer_decode(&d, &L, (const uint16_t *)x, T, (float *)y, (int32_t *)ids, (float *)w,
                         ws, wsb, NULL) == MOE_OK,
        "moe_layer_decode");
  CHECK(hipDeviceSynchronize() == hipSuccess, "synchronise");
  CHECK(hipMemcpy(yh, y, T * H * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(idh, ids, T * K * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(wh, w, T * K * 4, hipMemcpyDeviceToHost) == hipSuccess,
        "copy back");
  for (i = 0; i < (size_t)T * H; ++i) CHECK(yh[i] == 0.0f, "y == 0");
  for (i = 0; i < (size_t)T; ++i) {
    CHECK(idh[i * K] == 0 && idh[i * K + 1] == 1, "ids 0, 1 (ties to the lower index)");
    CHECK(wh[i * K] == 0.5f && wh[i * K + 1] == 0.5f, "weights 1/K");
  }
  {
    int32_t err = -1;
    CHECK(moe_get_device_error(ws, NULL, &err) == MOE_OK && err == 0, "no device error");
  }
  /* invalid arguments are refused before anything is enqueued */
  CHECK(moe_layer_decode(&d, &L, (const uint16_t *)x, T, (float *)y, NULL, NULL, ws, wsb - 1,
                         NULL) == MOE_ERR_WORKSPACE,
        "small workspace refused");
  hipFree(experts);
  hipFree(shared);
  hipFree(router);
  hipFree(x);
  hipFree(y);
  hipFree(ids);
  hipFree(w);
  hipFree(ws);
  return 0;
}
#endif

#ifdef MOE_C_GPU
/* Two layers of one token in the multi-layer kernel (full shape, 4 experts),
 * plain, and chained through the residual with the entry point that takes no
 * workspace: with zero weights y = 0, so the residual comes back unchanged. */
static int stack_checks(void) {
  const moe_dims d = {4096, 1024, 4, 4, 64, 4, 1};
  const size_t blob = moe_expert_bytes(&d), H = 4096, K = 4, NL = 2;
  const size_t wsb = moe_workspace_bytes(&d, 1);
  void *experts = NULL, *shared = NULL, *router = NULL, *x = NULL, *y = NULL, *ids = NULL,
       *w = NULL, *ws = NULL, *r = NULL;
  static float yh[2 * 4096], rh[4096], rback[4096];
  static uint16_t xh[2 * 4096];
  float wh[2 * 4];
  int32_t idh[2 * 4];
  size_t i;
  moe_layer L[2];
  CHECK(hipMalloc(&experts, 4 * blob) == hipSuccess && hipMalloc(&shared, blob) == hipSuccess &&
            hipMalloc(&router, 4 * H * 2) == hipSuccess && hipMalloc(&x, NL * H * 2) == hipSuccess &&
            hipMalloc(&y, NL * H * 4) == hipSuccess && hipMalloc(&ids, NL * K * 4) == hipSuccess &&
            hipMalloc(&w, NL * K * 4) == hipSuccess && hipMalloc(&ws, wsb) == hipSuccess &&
            hipMalloc(&r, H * 4) == hipSuccess,
        "hipMalloc (stack)");
  CHECK(hipMemset(experts, 0, 4 * blob) == hipSuccess && hipMemset(shared, 0, blob) == hipSuccess &&
            hipMemset(router, 0, 4 * H * 2) == hipSuccess && hipMemset(ws, 0, wsb) == hipSuccess,
        "hipMemset (stack)");
  for (i = 0; i < NL * H; ++i) xh[i] = (uint16_t)(0x3F80u + (i % 5));
  for (i = 0; i < H; ++i) rh[i] = (float)((int)(i % 11) - 5) * 0.25f;
  CHECK(hipMemcpy(x, xh, NL * H * 2, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(r, rh, H * 4, hipMemcpyHostToDevice) == hipSuccess,
        "copy x, r");
  for (i = 0; i < NL; ++i) {
    L[i].router = (const uint16_t *)router;
    L[i].experts = (const uint8_t *)experts;
    L[i].expert_stride = (int64_t)blob;
    L[i].shared = (const uint8_t *)shared;
  }
  CHECK(moe_stack_decode(&d, L, (int32_t)NL, (const uint16_t *)x, (float *)y, (int32_t *)ids,
                         (float *)w, ws, wsb, NULL) == MOE_OK,
        "moe_stack_decode");
  CHECK(hipDeviceSynchronize() == hipSuccess, "synchronise (stack)");
  CHECK(hipMemcpy(yh, y, NL * H * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(idh, ids, NL * K * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(wh, w, NL * K * 4, hipMemcpyDeviceToHost) == hipSuccess,
        "copy back (stack)");
  for (i = 0; i < NL * H; ++i) CHECK(yh[i] == 0.0f, "stack y == 0");
  for (i = 0; i < NL * K; ++i) {
    CHECK(idh[i] == (int32_t)(i % K), "stack ids 0..3");
    CHECK(wh[i] == 0.25f, "stack weights 1/4");
  }
  CHECK(moe_stack_decode_residual_noalloc(&d, L, (int32_t)NL, (float *)r, NULL, NULL,
                                          (int32_t *)ids, NULL, NULL) == MOE_OK,
        "moe_stack_decode_residual_noalloc");
  CHECK(hipDeviceSynchronize() == hipSuccess, "synchronise (residual)");
  CHECK(hipMemcpy(rback, r, H * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(idh, ids, NL * K * 4, hipMemcpyDeviceToHost) == hipSuccess,
        "copy back (residual)");
  for (i = 0; i < H; ++i) CHECK(rback[i] == rh[i], "residual unchanged (r += 0)");
  for (i = 0; i < NL * K; ++i) CHECK(idh[i] == (int32_t)(i % K), "residual ids 0..3");
  {
    int32_t err = -1;
    CHECK(moe_get_device_error(ws, NULL, &err) == MOE_OK && err == 0, "no device error (stack)");
  }
  hipFree(experts);
  hipFree(shared);
  hipFree(router);
  hipFree(x);
  hipFree(y);
  hipFree(ids);
  hipFree(w);
  hipFree(ws);
  hipFree(r);
  return 0;
}
#endif

int main(int argc, char **argv) {
  if (host_checks()) return 1;
#ifdef MOE_C_GPU
  if (argc > 1 && strcmp(argv[1], "gpu") == 0) {
    int T;
    for (T = 1; T <= 4; T += 3)
      if (gpu_checks(T)) return 1;
    if (stack_checks()) return 1;
  }
#else
  (void)argc;
  (void)argv;
#endif
  printf("ok\n");
  return 0;
}
