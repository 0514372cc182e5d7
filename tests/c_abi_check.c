/* A plain C99 caller of libgqa: the header compiles as C, the library links, and the host-only
 * calls answer (no GPU work: the argument checks fail before anything is enqueued). */
#include <stdio.h>

#include "gqa.h"

int main(void) {
  gqa_problem p = {1, 4, 2, 128, 64, 0.125f, 1, 0, 0, GQA_BF16};
  const int64_t pairs = gqa_visible_pairs(&p); /* causal: S (S + 1) / 2 */
  gqa_problem bad = p;
  bad.G = 3; /* H % G != 0 */
  const int st = gqa_attn_fwd(&bad, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
  printf("abi %d pairs %lld status %s\n", gqa_abi_version(), (long long)pairs, gqa_status_str(st));
  return (gqa_abi_version() == GQA_ABI_VERSION && pairs == 128 * 129 / 2 && st == GQA_ERR_INVALID_ARG) ? 0 : 1;
}
