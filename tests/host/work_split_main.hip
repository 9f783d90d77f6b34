// Host build of the attention kernels' work split index math (attn_common.h),
// driven by tests/test_work_split.py.  Reads from stdin:
//   mode (0 = shared tiles, 1 = fixed splits, 2 = shared tiles with the
//   closed-form prefix of equal lengths), batch, Hkv, tile, W,
//   split_tokens, splits, then batch list lengths.
// Prints one line per piece "P w b g part e_begin e_end" and, for shared
// tiles, one line per segment "C b g first count" followed by the flags of
// share_meets for the count partials.
#include <cstdio>
#include <vector>

#include "attn_common.h"

// Stream-K pieces and combine lookups under the tile prefix `pre` (an array,
// or UniformPre when all lists have the same length).
template <typename Pre, typename LenFn>
void shared_tiles(const Pre &pre, int batch, int Hkv, int tile, int W, LenFn len) {
  for (int w = 0; w < W; ++w) {
    vg::ShareWalk s = vg::share_walk_begin(pre, batch, Hkv, w, W);
    while (s.t < s.t_end) {
      const vg::Piece p = vg::share_walk_next(s, pre, Hkv, tile, w, len);
      printf("P %d %d %d %d %d %d\n", w, p.b, p.g, p.part, p.e_begin, p.e_end);
    }
  }
  for (int b = 0; b < batch; ++b)
    for (int g = 0; g < Hkv; ++g) {
      int first, count;
      vg::combine_range(pre, batch, Hkv, W, b, g, first, count);
      printf("C %d %d %d %d", b, g, first, count);
      for (int j = 0; j < count; ++j)
        printf(" %d", (int)vg::share_meets(pre, batch, Hkv, W, first + j - (b * Hkv + g), b, g));
      printf("\n");
    }
}

int main() {
  int mode, batch, Hkv, tile, W, split_tokens, splits;
  if (scanf("%d %d %d %d %d %d %d", &mode, &batch, &Hkv, &tile, &W, &split_tokens, &splits) != 7) return 2;
  std::vector<int> lens(batch), pre(batch + 1, 0);
  for (int b = 0; b < batch; ++b) {
    if (scanf("%d", &lens[b]) != 1) return 2;
    pre[b + 1] = pre[b] + (lens[b] + tile - 1) / tile;
  }
  auto len = [&](int b) { return lens[b]; };
  if (mode == 1) {
    for (int w = 0; w < W; ++w) {
      const vg::Piece p = vg::fixed_piece(w, splits, split_tokens, Hkv, lens[w / splits / Hkv]);
      printf("P %d %d %d %d %d %d\n", w, p.b, p.g, p.part, p.e_begin, p.e_end);
    }
  } else if (mode == 2) {  // every list as long as the first one, closed-form prefix
    const vg::UniformPre up{(lens[0] + tile - 1) / tile};
    shared_tiles(up, batch, Hkv, tile, W, [&](int) { return lens[0]; });
  } else {
    shared_tiles(pre.data(), batch, Hkv, tile, W, len);
  }
  return 0;
}
