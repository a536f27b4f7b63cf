/* Calls the library from plain C99 through include/kda.h alone (no GPU needed):
 * workspace sizing and the argument checks every entry point runs before it
 * launches anything.  Prints "ok" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "failed: %s\n", what);
    ++failures;
  }
}

int main(void) {
  kda_dims d;
  memset(&d, 0, sizeof d);
  d.num_heads = 16;
  d.head_dim_k = 128;
  d.head_dim_v = 128;
  d.conv_width = 4;
  d.in_dtype = KDA_DTYPE_BF16;
  d.conv_act = KDA_ACT_SILU;
  d.precision = KDA_PREC_FP16;
  d.decay_shape = KDA_DECAY_PER_DIM;

  const size_t need = kda_prefill_workspace_bytes(&d, 1, 4096);
  expect(need > 0, "workspace bytes for a valid geometry");
  expect(kda_prefill_workspace_bytes(&d, 2, 4096) > need, "a second sequence adds a record slot");

  kda_dims bad = d;
  bad.head_dim_k = 96;
  expect(kda_prefill_workspace_bytes(&bad, 1, 4096) == 0, "no workspace for an unsupported d_k");

  /* decode with an unsupported d_k is refused before any launch, with a message */
  static float dummy[64] __attribute__((aligned(256)));
  void* a = dummy;
  int rc = kda_decode(&bad, 4, NULL, dummy, a, dummy, a, a, a, a, a, KDA_GATE_SAFE, -5.0f, dummy, NULL);
  expect(rc == KDA_E_GEOMETRY, "decode refuses d_k = 96");
  const char* msg = kda_last_error();
  expect(msg != NULL && msg[0] != 0, "an error leaves a message");

  /* an unknown gate mode and a safe gate without a negative finite bound */
  rc = kda_decode(&d, 4, NULL, dummy, a, dummy, a, a, a, a, a, 9, -5.0f, dummy, NULL);
  expect(rc == KDA_E_GATE, "decode refuses gate mode 9");
  rc = kda_decode(&d, 4, NULL, dummy, a, dummy, a, a, a, a, a, KDA_GATE_SAFE, 0.0f, dummy, NULL);
  expect(rc == KDA_E_GATE, "decode refuses lower bound 0");

  /* an unknown precision policy */
  kda_dims badp = d;
  badp.precision = 4;
  expect(kda_prefill_workspace_bytes(&badp, 1, 4096) == 0, "no workspace for precision 4");

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
