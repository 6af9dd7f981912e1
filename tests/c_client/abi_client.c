/* A C99 client of the library's C ABI (include/moe.h): compiled with
 * -std=c99 -pedantic -Werror, linked against libmoe.so and run on the host.
 * It calls the host-only entry points and argument checks that fail before
 * anything is launched, so it needs no GPU; taking every entry point's
 * address makes each declared symbol resolve at link time. */
#include <stdio.h>
#include <string.h>

#include "moe.h"

typedef void (*any_fn)(void);

int main(void) {
  const any_fn entry_points[] = {
      (any_fn)moe_workspace_size,       (any_fn)moe_expert_ffn_workspace_size,
      (any_fn)moe_route,                (any_fn)moe_dispatch,
      (any_fn)moe_expert_ffn,           (any_fn)moe_combine,
      (any_fn)moe_forward,              (any_fn)moe_block_forward,
      (any_fn)moe_attention_workspace_size, (any_fn)moe_gqa_attention,
      (any_fn)moe_attention_block_forward,  (any_fn)moe_aux_loss,
      (any_fn)moe_set_timing_events,    (any_fn)moe_last_error,
  };
  moe_shape s, bad;
  size_t ws, i;
  int32_t idx[4];
  float w[4];
  moe_status st;
  const char* msg;

  for (i = 0; i < sizeof entry_points / sizeof entry_points[0]; ++i)
    if (entry_points[i] == NULL) return 10;

  memset(&s, 0, sizeof s);
  s.T = 16;
  s.d = 4096;
  s.d_ff = 14336;
  s.E = 8;
  s.k = 2;
  s.act = MOE_BF16;
  s.wt = MOE_BF16;
  ws = moe_workspace_size(&s);
  if (ws == 0) return 1;

  bad = s;
  bad.k = 9; /* top-k outside 1..E */
  if (moe_workspace_size(&bad) != 0) return 2;
  st = moe_route(&bad, idx, w, NULL, NULL, idx, w, NULL);
  if (st != MOE_ERR_INVALID_ARG) return 3;
  msg = moe_last_error();
  if (msg == NULL || msg[0] == '\0') return 4;

  printf("workspace %lu bytes; k = 9 rejected: %s\n", (unsigned long)ws, msg);
  return 0;
}
