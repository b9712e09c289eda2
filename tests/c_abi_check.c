/* Uses the library from plain C (no Python, no GPU): host-side argument checks of the device calls,
 * and the host packer and capacity estimate, which compute on the host. Prints one line per check;
 * tests/test_c_abi.py compiles it with gcc and compares the output. */
#include <stdint.h>
#include <stdio.h>

#include "opd.h"

int main(void) {
  const size_t ws = opd_workspace_size();
  printf("workspace %zu\n", ws);
  printf("status %s\n", opd_status_string(OPD_ERR_NULL));
  /* device entry points reject bad arguments before any HIP call */
  float* fake = (float*)(uintptr_t)(1u << 24);
  opd_status_t s = opd_loss_fwd(NULL, fake, OPD_BF16, 4, 64, 64, 0.5f, 0.05f, fake, (int32_t*)fake, NULL, fake,
                                fake, ws, NULL);
  printf("fwd null z %d\n", (int)s);
  s = opd_loss_fwd(fake, fake, OPD_BF16, 4, 64, 64, 1.5f, 0.05f, fake, (int32_t*)fake, NULL, fake, fake, ws, NULL);
  printf("fwd alpha %d %s\n", (int)s, opd_last_error());
  s = opd_verify_sample(fake, fake, OPD_BF16, 4, 64, 64, NULL, NULL, NULL, NULL, 1.0f, NULL, NULL, NULL, fake, ws,
                        NULL);
  printf("sample null blocks %d\n", (int)s);
  /* host scheduling */
  const int32_t lengths[6] = {8, 16, 5, 9, 7, 1};
  int32_t selected[6], offsets[7], packed[6], n_sel = -1;
  int64_t rows = -1;
  s = opd_pack_first_fit(lengths, 6, 20, 0, selected, offsets, packed, &n_sel, &rows);
  printf("pack %d n=%d rows=%lld sel=", (int)s, (int)n_sel, (long long)rows);
  for (int i = 0; i < n_sel; ++i) printf("%d%s", (int)selected[i], i + 1 < n_sel ? "," : "");
  printf(" off=");
  for (int i = 0; i <= n_sel; ++i) printf("%d%s", (int)offsets[i], i < n_sel ? "," : "");
  printf("\n");
  opd_capacity_t cap;
  int64_t budget = -1;
  s = opd_capacity_init(&cap, 0.5);
  printf("cap init %d\n", (int)s);
  opd_capacity_observe(&cap, 4000.0, &budget);
  printf("cap %lld", (long long)budget);
  opd_capacity_observe(&cap, 2000.0, &budget);
  printf(" %lld", (long long)budget);
  opd_capacity_observe(&cap, 2001.0, &budget);
  printf(" %lld\n", (long long)budget);
  s = opd_capacity_init(&cap, 1.5);
  printf("cap bad beta %d\n", (int)s);
  return 0;
}
