// Host driver for the split planner: reads one shape per line from stdin,
//   B Hq Hkv D max_blocks_per_seq block_size dtype requested_splits kv_fp8
// and prints, per line, the status code and the plan
//   status S P NH NT Pw HS
// (zeros after a failing status). Built with g++ against the planner source
// alone; it touches no GPU.
#include <stdio.h>

#include "../paged_gqa_decode_02_amd/csrc/pd_internal.h"

int main() {
  int B, Hq, Hkv, D, MB, bs, dtype, req, fp8;
  while (scanf("%d %d %d %d %d %d %d %d %d", &B, &Hq, &Hkv, &D, &MB, &bs, &dtype, &req, &fp8) ==
         9) {
    pd::Shape s{B, Hq, Hkv, D, MB, bs, dtype};
    pd::Plan p{};
    const int st = pd::make_plan(s, req, &p, fp8 != 0);
    if (st != 0) p = pd::Plan{};
    printf("%d %d %d %d %d %d %d\n", st, p.splits, p.partition_tokens, p.heads_per_group,
           p.slices, p.wave_tokens, p.head_split);
  }
  return 0;
}
