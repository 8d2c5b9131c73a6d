// Host-side check of the decode merge's head placement (merge_head_of in
// csrc/common.hpp): for every KV-head count the library accepts up to 64
// (0 included, the value the merge-only entry point passes) and every group
// size g in {1, 2, 4, 8, 16}, the map of merge workgroup x -> q head must be
// a bijection of [0, n_q_heads); for a multiple of 8 KV heads it must also
// place head h on the XCD slot (x mod 8) that wrote KV head h / g, i.e.
// (h / g) mod 8 == x mod 8; any other count must keep the identity.
// Compiled for the host only; prints one line and returns 0 on success.
#include <stdio.h>

#include <vector>

#include "common.hpp"

int main() {
  int checked = 0;
  for (int hkv = 0; hkv <= 64; ++hkv) {
    for (int g : {1, 2, 4, 8, 16}) {
      // hkv = 0: the merge-only path, which knows only n_q_heads
      const int hq = hkv == 0 ? 8 * g : hkv * g;
      std::vector<int> seen(hq, 0);
      for (int x = 0; x < hq; ++x) {
        const int h = pkv::merge_head_of(x, hq, hkv);
        if (h < 0 || h >= hq) {
          printf("FAIL out of range: hkv %d g %d x %d -> %d\n", hkv, g, x, h);
          return 1;
        }
        if (seen[h]++) {
          printf("FAIL not injective: hkv %d g %d x %d -> %d\n", hkv, g, x, h);
          return 1;
        }
        const bool placed = hkv > 0 && hkv % 8 == 0;
        if (placed && (h / g) % 8 != x % 8) {
          printf("FAIL placement: hkv %d g %d x %d -> %d\n", hkv, g, x, h);
          return 1;
        }
        if (!placed && h != x) {
          printf("FAIL identity: hkv %d g %d x %d -> %d\n", hkv, g, x, h);
          return 1;
        }
      }
      ++checked;
    }
  }
  printf("merge_head_of ok: %d (n_kv_heads, g) pairs\n", checked);
  return 0;
}
