// Host build of the attention kernels' work split index math (attn_common.h),
// driven by tests/test_work_split.py.  Reads from stdin:
//   mode (0 = shared tiles, 1 = fixed splits), batch, Hkv, tile, W,
//   split_tokens, splits, then batch list lengths.
// Prints one line per piece "P w b g part e_begin e_end" and, for shared
// tiles, one line per segment "C b g first count" followed by the flags of
// share_meets for the count partials.
#include <cstdio>
#include <vector>

#include "attn_common.h"

int main() {
  int mode, batch, Hkv, tile, W, split_tokens, splits;
  if (scanf("%d %d %d %d %d %d %d", &mode, &batch, &Hkv, &tile, &W, &split_tokens, &splits) != 7) return 2;
  std::vector<int> lens(batch), pre(batch + 1, 0);
  for (int b = 0; b < batch; ++b) {
    if (scanf("%d", &lens[b]) != 1) return 2;
    pre[b + 1] = pre[b] + (lens[b] + tile - 1) / tile;
  }
  auto len = [&](int b) { return lens[b]; };
  for (int w = 0; w < W; ++w) {
    if (mode == 1) {
      const vg::Piece p = vg::fixed_piece(w, splits, split_tokens, Hkv, lens[w / splits / Hkv]);
      printf("P %d %d %d %d %d %d\n", w, p.b, p.g, p.part, p.e_begin, p.e_end);
      continue;
    }
    vg::ShareWalk s = vg::share_walk_begin(pre.data(), batch, Hkv, w, W);
    while (s.t < s.t_end) {
      const vg::Piece p = vg::share_walk_next(s, pre.data(), Hkv, tile, w, len);
      printf("P %d %d %d %d %d %d\n", w, p.b, p.g, p.part, p.e_begin, p.e_end);
    }
  }
  if (mode == 0) {
    for (int b = 0; b < batch; ++b)
      for (int g = 0; g < Hkv; ++g) {
        int first, count;
        vg::combine_range(pre.data(), batch, Hkv, W, b, g, first, count);
        printf("C %d %d %d %d", b, g, first, count);
        for (int j = 0; j < count; ++j)
          printf(" %d", (int)vg::share_meets(pre.data(), batch, Hkv, W, first + j - (b * Hkv + g), b, g));
        printf("\n");
      }
  }
  return 0;
}
