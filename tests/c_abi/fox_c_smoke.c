/* fox_c_smoke.c - the attention path driven from plain C through include/fox.h, with device
 * memory from the HIP runtime and no Python or PyTorch in the process.
 *
 *   fox_c_smoke B H L D IN_DIR OUT_DIR
 *
 * Reads IN_DIR/{q,k,v,do}.bin (bf16, [B, H, L, D], raw little-endian) and IN_DIR/logf.bin
 * (fp32, [B, H, L]); runs fox_logf_cumsum, fox_attn_fwd (fp32 O) and fox_attn_bwd on the
 * default stream; writes OUT_DIR/{o,lse,dq,dk,dv,dlogf}.bin (fp32). Exits 0 on success, 1 with
 * a message on stderr on any failed call (a fox_status other than FOX_OK carries
 * fox_last_error()), 2 on bad arguments or files. Built by the package's build step. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fox.h"

static int read_file(const char* dir, const char* name, void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return fprintf(stderr, "cannot open %s\n", path), 0;
  const size_t got = fread(buf, 1, bytes, f);
  fclose(f);
  if (got != bytes) return fprintf(stderr, "%s: %zu of %zu bytes\n", path, got, bytes), 0;
  return 1;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return fprintf(stderr, "cannot create %s\n", path), 0;
  const size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

#define FOX_OK_(call)                                                                  \
  do {                                                                                 \
    fox_status s_ = (call);                                                            \
    if (s_ != FOX_OK) {                                                                \
      fprintf(stderr, "%s: %s (%s)\n", #call, fox_status_str(s_), fox_last_error());  \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s B H L D IN_DIR OUT_DIR\n", argv[0]);
    return 2;
  }
  const int64_t B = atoll(argv[1]), H = atoll(argv[2]), L = atoll(argv[3]), D = atoll(argv[4]);
  if (B < 1 || H < 1 || L < 1 || (D != 64 && D != 128) || B * H * L > (int64_t)1 << 26) {
    fprintf(stderr, "sizes out of range for this program\n");
    return 2;
  }
  const size_t n4 = (size_t)(B * H * L * D), n3 = (size_t)(B * H * L);
  const float scale = 1.0f / sqrtf((float)D);

  uint16_t* hq = malloc(n4 * 2);
  uint16_t* hk = malloc(n4 * 2);
  uint16_t* hv = malloc(n4 * 2);
  uint16_t* hdo = malloc(n4 * 2);
  float* hlf = malloc(n3 * 4);
  float* h4 = malloc(n4 * 4);
  float* h3 = malloc(n3 * 4);
  if (!hq || !hk || !hv || !hdo || !hlf || !h4 || !h3) return fprintf(stderr, "out of memory\n"), 2;
  if (!read_file(argv[5], "q.bin", hq, n4 * 2) || !read_file(argv[5], "k.bin", hk, n4 * 2) ||
      !read_file(argv[5], "v.bin", hv, n4 * 2) || !read_file(argv[5], "do.bin", hdo, n4 * 2) ||
      !read_file(argv[5], "logf.bin", hlf, n3 * 4))
    return 2;

  void *q, *k, *v, *dO, *ws;
  float *lf, *c, *o, *lse, *dq, *dk, *dv, *dlf;
  HIP_OK(hipMalloc(&q, n4 * 2));
  HIP_OK(hipMalloc(&k, n4 * 2));
  HIP_OK(hipMalloc(&v, n4 * 2));
  HIP_OK(hipMalloc(&dO, n4 * 2));
  HIP_OK(hipMalloc((void**)&lf, n3 * 4));
  HIP_OK(hipMalloc((void**)&c, n3 * 4));
  HIP_OK(hipMalloc((void**)&o, n4 * 4));
  HIP_OK(hipMalloc((void**)&lse, n3 * 4));
  HIP_OK(hipMalloc((void**)&dq, n4 * 4));
  HIP_OK(hipMalloc((void**)&dk, n4 * 4));
  HIP_OK(hipMalloc((void**)&dv, n4 * 4));
  HIP_OK(hipMalloc((void**)&dlf, n3 * 4));
  const size_t ws_bytes = fox_attn_bwd_workspace_bytes(B, H, L, D);
  if (ws_bytes == 0) return fprintf(stderr, "no workspace size for these sizes\n"), 1;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(q, hq, n4 * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, n4 * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, n4 * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dO, hdo, n4 * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(lf, hlf, n3 * 4, hipMemcpyHostToDevice));

  FOX_OK_(fox_logf_cumsum(lf, c, B * H, L, NULL));
  FOX_OK_(fox_attn_fwd(q, k, v, FOX_BF16, c, o, FOX_F32, lse, B, H, L, D, scale, FOX_CAUSAL,
                       NULL, NULL));
  FOX_OK_(fox_attn_bwd(q, k, v, FOX_BF16, c, o, lse, dO, dq, dk, dv, dlf, ws, ws_bytes, B, H, L,
                       D, scale, FOX_CAUSAL, NULL, NULL));
  HIP_OK(hipDeviceSynchronize());

  const struct { const char* name; const float* src; size_t n; } outs[] = {
      {"o.bin", o, n4}, {"lse.bin", lse, n3}, {"dq.bin", dq, n4},
      {"dk.bin", dk, n4}, {"dv.bin", dv, n4}, {"dlogf.bin", dlf, n3}};
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
    float* host = outs[i].n == n4 ? h4 : h3;
    HIP_OK(hipMemcpy(host, outs[i].src, outs[i].n * 4, hipMemcpyDeviceToHost));
    if (!write_file(argv[6], outs[i].name, host, outs[i].n * 4)) return 2;
  }
  hipFree(q); hipFree(k); hipFree(v); hipFree(dO); hipFree(ws);
  hipFree(lf); hipFree(c); hipFree(o); hipFree(lse); hipFree(dq); hipFree(dk); hipFree(dv);
  hipFree(dlf);
  free(hq); free(hk); free(hv); free(hdo); free(hlf); free(h4); free(h3);
  printf("fox_c_smoke ok\n");
  return 0;
}
