/* A plain C caller of the library's host-side entry points: the workspace
 * size and layout, the grouping capacity and argument validation.  None of
 * these calls touches the GPU.  Prints one line per figure, which the test
 * compares with what the Python binding reports. */
#include <stdio.h>
#include <string.h>

#include "moe_mi355x.h"

/* A Qwen3-30B-A3B-shaped layer (H=2048, E=128, top-8, I=768, bf16). */
static moe_problem layer(int64_t num_tokens) {
  moe_problem p;
  memset(&p, 0, sizeof p);
  p.num_tokens = num_tokens;
  p.hidden = 2048;
  p.num_experts = 128;
  p.top_k = 8;
  p.inter = 768;
  p.dtype = MOE_BF16;
  p.norm_topk_prob = 1;
  p.weight_layout = MOE_LAYOUT_BLOCKED;
  return p;
}

int main(void) {
  const int64_t tokens[] = {64, 4096};
  for (int i = 0; i < 2; ++i) {
    moe_problem p = layer(tokens[i]);
    size_t bytes = 0;
    moe_workspace_layout L;
    if (moe_workspace_size(&p, &bytes) != MOE_OK || moe_get_workspace_layout(&p, &L) != MOE_OK) {
      fprintf(stderr, "layout query failed: %s\n", moe_last_error());
      return 1;
    }
    if (L.total_bytes != bytes) return 2;
    printf("layout %lld %zu %lld %lld %lld %zu %zu\n", (long long)tokens[i], bytes, (long long)L.block_m,
           (long long)L.max_tiles, (long long)L.ids_products, L.act, L.y);
  }
  int64_t rows = 0, tiles = 0;
  if (moe_align_capacity(32768, 128, 320, &rows, &tiles) != MOE_OK) return 3;
  printf("capacity %lld %lld\n", (long long)rows, (long long)tiles);

  size_t bytes = 0;
  moe_problem bad = layer(4);
  bad.num_experts = 4;                               /* top_k = 8 > E */
  printf("top_k_above_E %d\n", moe_workspace_size(&bad, &bytes));
  bad = layer(4);
  bad.top_k = 33;                                    /* above the supported 32 */
  printf("top_k_above_limit %d\n", moe_workspace_size(&bad, &bytes));
  printf("null_problem %d\n", moe_workspace_size(NULL, &bytes));
  moe_problem p = layer(64);
  printf("forward_null_tensors %d\n",
         moe_forward(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  printf("last_error_set %d\n", moe_last_error()[0] != '\0');
  return 0;
}
