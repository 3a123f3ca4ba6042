/* A plain C99 caller of the library's C ABI: built with gcc -std=c99
 * -pedantic -Werror against include/moe.h and linked to libmoe.so by
 * tests/test_abi_c.py.  It calls only entry points that validate on the host
 * (no GPU needed) and prints one result per line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static moe_cfg decode16(void) {
  moe_cfg c;
  memset(&c, 0, sizeof c);
  c.T = 16;
  c.H = 7168;
  c.E = 256;
  c.k = 8;
  c.I = 2048;
  c.I_shared = 2048;
  c.score = MOE_SCORE_SIGMOID;
  c.act_dtype = MOE_BF16;
  c.w_dtype = MOE_BF16;
  c.quant_block = 128;
  c.routed_scale = 1.0f;
  c.n_group = 1;
  c.topk_group = 1;
  c.w_block_rows = 1;
  return c;
}

int main(void) {
  moe_cfg c = decode16();
  size_t bytes = 0, h = 0, hq = 0, hs = 0;
  int st = moe_workspace_size(&c, &bytes);
  printf("workspace_size %d %s %zu\n", st, moe_status_str(st), bytes);
  printf("workspace_bytes %zu\n", moe_workspace_bytes(&c));
  st = moe_workspace_ffn_h(&c, &h, &hq, &hs);
  printf("ffn_h %d %zu %d %d\n", st, h, hq == SIZE_MAX, hs == SIZE_MAX);
  c.k = 0;
  st = moe_workspace_size(&c, &bytes);
  printf("bad_cfg %d %s\n", st, moe_status_str(st));
  printf("last_error %s\n", moe_last_error()[0] ? "set" : "empty");
  c = decode16();
  /* validation fails before anything is enqueued: no GPU is touched */
  st = moe_forward(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  printf("forward_null_x %d %s\n", st, moe_status_str(st));
  return 0;
}
