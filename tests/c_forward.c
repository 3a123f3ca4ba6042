/* A plain C99 host program that runs the whole layer through the library's
 * C ABI with the HIP runtime alone (no Python, no torch): built and run by
 * tests/test_abi_c.py on a GPU.
 *
 *   c_forward DIR
 *
 * DIR/cfg.txt holds "T H E k I I_shared score act_dtype w_dtype quant_block
 * w_block_rows"; DIR/x.bin, wg.bin, bias.bin, w13.bin, w2.bin (and ws13.bin,
 * ws2.bin with a shared expert; w13s.bin, w2s.bin, ws13s.bin, ws2s.bin with
 * fp8 weights) hold the raw arrays.  Writes DIR/y.bin and DIR/idx.bin.  Exit
 * status 0 on success; otherwise the failing call is printed. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

static const char* g_dir;

static void* load(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  void* host = malloc(bytes);
  if (!host || fread(host, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
  fclose(f);
  void* dev = NULL;
  if (hipMalloc(&dev, bytes) != hipSuccess || hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device copy of %s failed\n", name);
    exit(2);
  }
  free(host);
  return dev;
}

static void save(const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  void* host = malloc(bytes);
  if (!host || hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "copy back of %s failed\n", name);
    exit(2);
  }
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
  free(host);
}

int main(int argc, char** argv) {
  if (argc != 2) { fprintf(stderr, "usage: c_forward DIR\n"); return 2; }
  g_dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/cfg.txt", g_dir);
  FILE* f = fopen(path, "r");
  moe_cfg c;
  memset(&c, 0, sizeof c);
  if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d", &c.T, &c.H, &c.E, &c.k, &c.I, &c.I_shared, &c.score,
                   &c.act_dtype, &c.w_dtype, &c.quant_block, &c.w_block_rows) != 11) {
    fprintf(stderr, "bad cfg.txt\n");
    return 2;
  }
  fclose(f);
  c.routed_scale = 1.0f;
  c.n_group = 1;
  c.topk_group = 1;
  const size_t ab = c.act_dtype == MOE_F32 ? 4 : 2;
  const size_t wb = c.w_dtype == MOE_F32 ? 4 : (c.w_dtype == MOE_BF16 ? 2 : 1);
  const int fp8 = c.w_dtype == MOE_FP8_E4M3;
  const size_t T = c.T, H = c.H, E = c.E, I = c.I, k = c.k, qb = c.quant_block, br = c.w_block_rows;
  void* x = load("x.bin", T * H * ab);
  void* wg = load("wg.bin", E * H * ab);
  float* bias = (float*)load("bias.bin", E * 4);
  moe_weights w;
  memset(&w, 0, sizeof w);
  w.w13 = load("w13.bin", E * 2 * I * H * wb);
  w.w2 = load("w2.bin", E * H * I * wb);
  if (fp8) {
    w.w13_scale = (const float*)load("w13s.bin", E * (2 * I / br) * (H / qb) * 4);
    w.w2_scale = (const float*)load("w2s.bin", E * (H / br) * (I / qb) * 4);
  }
  if (c.I_shared > 0) {
    w.ws13 = load("ws13.bin", 2 * I * H * wb);
    w.ws2 = load("ws2.bin", H * I * wb);
    if (fp8) {
      w.ws13_scale = (const float*)load("ws13s.bin", (2 * I / br) * (H / qb) * 4);
      w.ws2_scale = (const float*)load("ws2s.bin", (H / br) * (I / qb) * 4);
    }
  }
  const size_t ws_bytes = moe_workspace_bytes(&c);
  if (ws_bytes == 0) { fprintf(stderr, "moe_workspace_bytes: %s\n", moe_last_error()); return 1; }
  void *ws = NULL, *y = NULL, *idx = NULL;
  if (hipMalloc(&ws, ws_bytes) != hipSuccess || hipMemset(ws, 0, ws_bytes) != hipSuccess ||
      hipMalloc(&y, T * H * ab) != hipSuccess || hipMalloc(&idx, T * k * 4) != hipSuccess) {
    fprintf(stderr, "allocation failed\n");
    return 2;
  }
  const int st = moe_forward(&c, x, wg, bias, &w, y, (int32_t*)idx, NULL, NULL, ws, ws_bytes, NULL);
  if (st != MOE_OK) { fprintf(stderr, "moe_forward: %s (%s)\n", moe_status_str(st), moe_last_error()); return 1; }
  if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "hipDeviceSynchronize failed\n"); return 1; }
  save("y.bin", y, T * H * ab);
  save("idx.bin", idx, T * k * 4);
  printf("ok\n");
  return 0;
}
