/*
 * Plain C user of libmoe_route.so: no Python, no torch.
 *
 *   abi_smoke         host-side checks only (no device is touched): version,
 *                     status strings, and argument validation.
 *   abi_smoke gpu     also runs route -> dispatch -> combine on a small
 *                     problem in device memory and checks what the method
 *                     guarantees: counts sum to T*k, offsets are their
 *                     exclusive scan, pair_row is a bijection onto [0, T*k)
 *                     with row_token as its inverse, every dispatched row is
 *                     a bit copy of its token, and combine over the dispatched
 *                     rows (identity experts) returns the input; then
 *                     moe_route_dispatch and moe_dispatch_noalloc against the
 *                     separate calls, byte for byte.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_route.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static void host_checks(void) {
  void* p16 = (void*)(uintptr_t)0x10000; /* fake, never dereferenced */
  CHECK(moe_abi_version() == MOE_ABI_VERSION);
  CHECK(strcmp(moe_strerror(MOE_OK), "ok") == 0);
  CHECK(moe_strerror(-12345) != NULL);
  CHECK(moe_route_topk(p16, 4, 8, 9, p16, p16, NULL) == MOE_ERR_INVALID_ARG);
  CHECK(moe_route_topk(NULL, 0, 8, 2, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_dispatch_recv(p16, p16, 16, 255, 2, p16, 32, NULL) == MOE_ERR_ALIGNMENT);
  CHECK(moe_dispatch_recv(p16, p16, 16, 256, 2, p16, 31, NULL) == MOE_ERR_CAPACITY);
  CHECK(moe_combine(p16, p16, p16, 16, 256, 33, 1024, p16, NULL) == MOE_ERR_INVALID_ARG);
  CHECK(moe_dispatch_workspace_bytes(8192, 256, 8) > 0);
  CHECK(moe_route_dispatch_workspace_bytes(128, 256, 8) == 256);
  CHECK(moe_route_dispatch(p16, p16, 16, 8, 2, 1, 1, 256, 1, p16, p16, p16, p16, p16, p16, NULL, p16,
                           32, NULL, 0, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_route_dispatch(p16, p16, 16, 8, 2, 3, 1, 256, 1, p16, p16, p16, p16, p16, p16, NULL, p16,
                           32, p16, 256, NULL) == MOE_ERR_INVALID_ARG); /* E % n_group != 0 */
  CHECK(moe_dispatch_noalloc(p16, p16, 16, 8, 2, 256, 1, p16, p16, p16, p16, NULL, p16, 31, NULL) ==
        MOE_ERR_CAPACITY);
  CHECK(moe_dispatch_noalloc(NULL, NULL, 0, 8, 2, 256, 1, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                             NULL) == MOE_OK);
}

static uint16_t bf16_of(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* A failed HIP call ends the GPU checks: later steps would pass unset
 * device pointers to the library. */
#define HIPCHECK(x)                                                   \
  do {                                                                \
    if ((x) != hipSuccess) {                                          \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #x);   \
      ++failures;                                                     \
      return;                                                         \
    }                                                                 \
  } while (0)

static void gpu_checks(void) {
  enum { T = 300, E = 16, K = 4, H = 256, R = 4 };
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    fprintf(stderr, "FAIL %s:%d: no GPU visible\n", __FILE__, __LINE__);
    ++failures;
    return;
  }
  const int P = T * K;
  float* logits = malloc(sizeof(float) * T * E);
  uint16_t* x = malloc(2 * T * H);
  uint32_t s = 12345u;
  for (int i = 0; i < T * E; ++i) {
    s = s * 1664525u + 1013904223u;
    logits[i] = (float)((s >> 8) & 0xFFFF) / 4096.0f - 8.0f;
  }
  for (int i = 0; i < T * H; ++i) {
    s = s * 1664525u + 1013904223u;
    x[i] = bf16_of((float)((int)(s >> 16) - 32768) / 8192.0f);
  }
  float *d_logits, *d_w;
  int32_t *d_idx, *d_counts, *d_off, *d_pr, *d_rt, *d_roff;
  void *d_x, *d_buf, *d_out, *d_ws = NULL;
  size_t wsb = moe_dispatch_workspace_bytes(T, E, K);
  HIPCHECK(hipMalloc((void**)&d_logits, sizeof(float) * T * E));
  HIPCHECK(hipMalloc((void**)&d_w, sizeof(float) * P));
  HIPCHECK(hipMalloc((void**)&d_idx, sizeof(int32_t) * P));
  HIPCHECK(hipMalloc((void**)&d_counts, sizeof(int32_t) * E));
  HIPCHECK(hipMalloc((void**)&d_off, sizeof(int32_t) * (E + 1)));
  HIPCHECK(hipMalloc((void**)&d_pr, sizeof(int32_t) * P));
  HIPCHECK(hipMalloc((void**)&d_rt, sizeof(int32_t) * P));
  HIPCHECK(hipMalloc((void**)&d_roff, sizeof(int32_t) * (R + 1)));
  HIPCHECK(hipMalloc(&d_x, 2 * T * H));
  HIPCHECK(hipMalloc(&d_buf, 2 * (size_t)P * H));
  HIPCHECK(hipMalloc(&d_out, 2 * T * H));
  if (wsb) HIPCHECK(hipMalloc(&d_ws, wsb));
  HIPCHECK(hipMemcpy(d_logits, logits, sizeof(float) * T * E, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_x, x, 2 * T * H, hipMemcpyHostToDevice));

  CHECK(moe_route_topk(d_logits, T, E, K, d_idx, d_w, NULL) == MOE_OK);
  CHECK(moe_dispatch(d_idx, d_x, T, E, K, H, R, d_counts, d_off, d_pr, d_rt, d_roff, d_buf, P, d_ws,
                     wsb, NULL) == MOE_OK);
  CHECK(moe_combine(d_buf, d_pr, d_w, T, H, K, P, d_out, NULL) == MOE_OK);
  HIPCHECK(hipDeviceSynchronize());

  int32_t* idx = malloc(sizeof(int32_t) * P);
  int32_t* counts = malloc(sizeof(int32_t) * E);
  int32_t* off = malloc(sizeof(int32_t) * (E + 1));
  int32_t* pr = malloc(sizeof(int32_t) * P);
  int32_t* rt = malloc(sizeof(int32_t) * P);
  uint16_t* buf = malloc(2 * (size_t)P * H);
  uint16_t* out = malloc(2 * T * H);
  HIPCHECK(hipMemcpy(idx, d_idx, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(counts, d_counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(off, d_off, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(pr, d_pr, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(rt, d_rt, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(buf, d_buf, 2 * (size_t)P * H, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(out, d_out, 2 * T * H, hipMemcpyDeviceToHost));

  /* moe_route_dispatch (route and send in one launch at this size) into
     fresh buffers: the same bytes as the three separate calls. */
  {
    float* d_w2;
    int32_t *d_idx2, *d_counts2, *d_off2, *d_pr2, *d_rt2, *d_roff2;
    void *d_buf2, *d_ws2;
    const size_t rwsb = moe_route_dispatch_workspace_bytes(T, E, K);
    HIPCHECK(hipMalloc((void**)&d_w2, sizeof(float) * P));
    HIPCHECK(hipMalloc((void**)&d_idx2, sizeof(int32_t) * P));
    HIPCHECK(hipMalloc((void**)&d_counts2, sizeof(int32_t) * E));
    HIPCHECK(hipMalloc((void**)&d_off2, sizeof(int32_t) * (E + 1)));
    HIPCHECK(hipMalloc((void**)&d_pr2, sizeof(int32_t) * P));
    HIPCHECK(hipMalloc((void**)&d_rt2, sizeof(int32_t) * P));
    HIPCHECK(hipMalloc((void**)&d_roff2, sizeof(int32_t) * (R + 1)));
    HIPCHECK(hipMalloc(&d_buf2, 2 * (size_t)P * H));
    HIPCHECK(hipMalloc(&d_ws2, rwsb));
    HIPCHECK(hipMemset(d_ws2, 0, rwsb)); /* the workspace starts zeroed */
    for (int rep = 0; rep < 2; ++rep)
      CHECK(moe_route_dispatch(d_logits, d_x, T, E, K, 1, 1, H, R, d_idx2, d_w2, d_counts2, d_off2,
                               d_pr2, d_rt2, d_roff2, d_buf2, P, d_ws2, rwsb, NULL) == MOE_OK);
    HIPCHECK(hipDeviceSynchronize());
    int32_t* i2 = malloc(sizeof(int32_t) * P);
    int32_t* r2 = malloc(sizeof(int32_t) * P);
    uint16_t* b2 = malloc(2 * (size_t)P * H);
    unsigned char* wsh = malloc(rwsb);
    HIPCHECK(hipMemcpy(i2, d_idx2, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
    CHECK(memcmp(i2, idx, sizeof(int32_t) * P) == 0);
    HIPCHECK(hipMemcpy(i2, d_pr2, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
    CHECK(memcmp(i2, pr, sizeof(int32_t) * P) == 0);
    HIPCHECK(hipMemcpy(r2, d_rt2, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
    CHECK(memcmp(r2, rt, sizeof(int32_t) * P) == 0);
    HIPCHECK(hipMemcpy(b2, d_buf2, 2 * (size_t)P * H, hipMemcpyDeviceToHost));
    CHECK(memcmp(b2, buf, 2 * (size_t)P * H) == 0);
    HIPCHECK(hipMemcpy(wsh, d_ws2, rwsb, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < rwsb; ++i) CHECK(wsh[i] == 0); /* and every call leaves it so */
    free(i2); free(r2); free(b2); free(wsh);
    hipFree(d_w2); hipFree(d_idx2); hipFree(d_counts2); hipFree(d_off2); hipFree(d_pr2);
    hipFree(d_rt2); hipFree(d_roff2); hipFree(d_buf2); hipFree(d_ws2);
  }

  /* moe_dispatch_noalloc on a batch that needs the multi-block send (its
     scratch in the library's own device array), twice: the same bytes as
     moe_dispatch with a caller workspace. */
  {
    enum { T2 = 2048, E2 = 64, K2 = 4, H2 = 64, R2 = 8, P2 = T2 * K2 };
    float* lg2 = malloc(sizeof(float) * T2 * E2);
    uint16_t* x2 = malloc(2 * T2 * H2);
    for (int i = 0; i < T2 * E2; ++i) {
      s = s * 1664525u + 1013904223u;
      lg2[i] = (float)((s >> 8) & 0xFFFF) / 4096.0f - 8.0f;
    }
    for (int i = 0; i < T2 * H2; ++i) {
      s = s * 1664525u + 1013904223u;
      x2[i] = bf16_of((float)((int)(s >> 16) - 32768) / 8192.0f);
    }
    float *d_lg, *d_wt;
    int32_t *d_id, *d_c[2], *d_o[2], *d_p[2], *d_r[2], *d_ro[2];
    void *d_xx, *d_b[2], *d_wsp;
    const size_t wsb2 = moe_dispatch_workspace_bytes(T2, E2, K2);
    CHECK(wsb2 > 0);
    HIPCHECK(hipMalloc((void**)&d_lg, sizeof(float) * T2 * E2));
    HIPCHECK(hipMalloc((void**)&d_wt, sizeof(float) * P2));
    HIPCHECK(hipMalloc((void**)&d_id, sizeof(int32_t) * P2));
    HIPCHECK(hipMalloc(&d_xx, 2 * T2 * H2));
    HIPCHECK(hipMalloc(&d_wsp, wsb2));
    for (int v = 0; v < 2; ++v) {
      HIPCHECK(hipMalloc((void**)&d_c[v], sizeof(int32_t) * E2));
      HIPCHECK(hipMalloc((void**)&d_o[v], sizeof(int32_t) * (E2 + 1)));
      HIPCHECK(hipMalloc((void**)&d_p[v], sizeof(int32_t) * P2));
      HIPCHECK(hipMalloc((void**)&d_r[v], sizeof(int32_t) * P2));
      HIPCHECK(hipMalloc((void**)&d_ro[v], sizeof(int32_t) * (R2 + 1)));
      HIPCHECK(hipMalloc(&d_b[v], 2 * (size_t)P2 * H2));
    }
    HIPCHECK(hipMemcpy(d_lg, lg2, sizeof(float) * T2 * E2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_xx, x2, 2 * T2 * H2, hipMemcpyHostToDevice));
    CHECK(moe_route_topk(d_lg, T2, E2, K2, d_id, d_wt, NULL) == MOE_OK);
    CHECK(moe_dispatch(d_id, d_xx, T2, E2, K2, H2, R2, d_c[0], d_o[0], d_p[0], d_r[0], d_ro[0],
                       d_b[0], P2, d_wsp, wsb2, NULL) == MOE_OK);
    for (int rep = 0; rep < 2; ++rep)
      CHECK(moe_dispatch_noalloc(d_id, d_xx, T2, E2, K2, H2, R2, d_c[1], d_o[1], d_p[1], d_r[1],
                                 d_ro[1], d_b[1], P2, NULL) == MOE_OK);
    HIPCHECK(hipDeviceSynchronize());
    const size_t sizes[6] = {sizeof(int32_t) * E2, sizeof(int32_t) * (E2 + 1), sizeof(int32_t) * P2,
                             sizeof(int32_t) * P2, sizeof(int32_t) * (R2 + 1), 2 * (size_t)P2 * H2};
    unsigned char* h0 = malloc(sizes[5]);
    unsigned char* h1 = malloc(sizes[5]);
    void* a0[6] = {d_c[0], d_o[0], d_p[0], d_r[0], d_ro[0], d_b[0]};
    void* a1[6] = {d_c[1], d_o[1], d_p[1], d_r[1], d_ro[1], d_b[1]};
    for (int i = 0; i < 6; ++i) {
      HIPCHECK(hipMemcpy(h0, a0[i], sizes[i], hipMemcpyDeviceToHost));
      HIPCHECK(hipMemcpy(h1, a1[i], sizes[i], hipMemcpyDeviceToHost));
      CHECK(memcmp(h0, h1, sizes[i]) == 0);
    }
    free(h0); free(h1); free(lg2); free(x2);
    hipFree(d_lg); hipFree(d_wt); hipFree(d_id); hipFree(d_xx); hipFree(d_wsp);
    for (int v = 0; v < 2; ++v) {
      hipFree(d_c[v]); hipFree(d_o[v]); hipFree(d_p[v]); hipFree(d_r[v]); hipFree(d_ro[v]);
      hipFree(d_b[v]);
    }
  }

  long total = 0;
  for (int e = 0; e < E; ++e) {
    total += counts[e];
    CHECK(off[e + 1] - off[e] == counts[e]);
  }
  CHECK(total == P && off[0] == 0 && off[E] == P);
  char* seen = calloc(P, 1);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int e = idx[t * K + j], r = pr[t * K + j];
      CHECK(e >= 0 && e < E && r >= off[e] && r < off[e + 1] && !seen[r]);
      seen[r] = 1;
      CHECK(rt[r] == t);
      CHECK(memcmp(buf + (size_t)r * H, x + (size_t)t * H, 2 * H) == 0);
    }
  for (int i = 0; i < T * H; ++i) CHECK(out[i] == (x[i] == 0x8000 ? 0 : x[i]));
  free(seen);
  free(idx); free(counts); free(off); free(pr); free(rt); free(buf); free(out);
  hipFree(d_logits); hipFree(d_w); hipFree(d_idx); hipFree(d_counts); hipFree(d_off);
  hipFree(d_pr); hipFree(d_rt); hipFree(d_roff); hipFree(d_x); hipFree(d_buf); hipFree(d_out);
  if (d_ws) hipFree(d_ws);
  free(logits); free(x);
}

int main(int argc, char** argv) {
  host_checks();
  if (argc > 1 && strcmp(argv[1], "gpu") == 0) gpu_checks();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_smoke ok%s\n", argc > 1 ? " (gpu)" : "");
  return 0;
}
