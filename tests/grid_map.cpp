// Host program for test_grid_maps.py: prints the bwd_kv grid that kv_grid_blocks / kv_grid_item
// (saf_internal.h) define for one shape.  Arguments: B Hkv n_kv_ord nkb rep_sec.
// Output: the block count, then one line "ok slot key_block" per block.
#include <cstdio>
#include <cstdlib>

#include "saf_internal.h"

int main(int argc, char** argv) {
  if (argc != 6) return 2;
  const int B = atoi(argv[1]), Hkv = atoi(argv[2]), nko = atoi(argv[3]), nkb = atoi(argv[4]);
  const bool rep_sec = atoi(argv[5]) != 0;
  const int n = saf::kv_grid_blocks(B, Hkv, nko, nkb, rep_sec);
  printf("%d\n", n);
  for (int x = 0; x < n; ++x) {
    int bh = -1, kb = -1;
    const bool ok = saf::kv_grid_item(B, Hkv, nko, nkb, x, bh, kb, rep_sec);
    printf("%d %d %d\n", ok ? 1 : 0, bh, kb);
  }
  return 0;
}
