// Host program for test_grid_maps.py: the indexing of the stored dS (saf_internal.h: ord_rank,
// ds_bytes).  Arguments: B T mask, mask a string of H characters ('1' = replaced head).
// Output: "n_ord ds_bytes", then one line "h rank" per ordinary head.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "saf_internal.h"

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int B = atoi(argv[1]), T = atoi(argv[2]);
  const char* mask = argv[3];
  const int H = (int)strlen(mask);
  if (H < 1 || H > saf::kMaxHeads) return 2;
  uint64_t rep[saf::kMaxHeads / 64] = {};
  int n_ord = 0;
  for (int h = 0; h < H; ++h) {
    if (mask[h] == '1') rep[h >> 6] |= 1ull << (h & 63);
    else ++n_ord;
  }
  printf("%d %zu\n", n_ord, saf::ds_bytes(B, n_ord, T));
  for (int h = 0; h < H; ++h)
    if (!saf::is_replaced(rep, h)) printf("%d %d\n", h, saf::ord_rank(rep, h));
  return 0;
}
