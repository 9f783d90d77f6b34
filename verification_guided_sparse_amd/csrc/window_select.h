// window_select.h -- query-agnostic selection: the first n_sink prefix positions
// (attention sinks) and the most recent positions, k_b in all, emitted in the
// same form as the exact top-k (ascending positions, page-size-1 slots, count)
// so that the same sparse draft kernel consumes either list.  It reads no
// scores: its cost is one tiny launch, the baseline that the pages set beside
// query-aware selection.
#pragma once

#include "vg_device.h"

namespace vg {

struct WindowArgs {
  const int32_t *prefix_len, *k, *page_table;  // [B], [B], [B][max_pages]
  int32_t *sel_pos, *sel_slot, *sel_count;     // [B][max_k], [B][max_k] (nullable), [B]
  int32_t max_prefix, max_k, n_sink, page_size, max_pages;
};

__global__ __launch_bounds__(256) void window_select_kernel(WindowArgs a) {
  const int b = blockIdx.y;
  // lengths are clamped to what the buffers hold, so a bad length cannot
  // turn into an out-of-bounds write
  const int P = min(max(a.prefix_len[b], 0), a.max_prefix);
  const int kk = min(min(max(a.k[b], 0), P), a.max_k);
  const int s = min(a.n_sink, kk);
  const size_t row = (size_t)b * a.max_k;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < kk; i += gridDim.x * blockDim.x) {
    // [0, s) then [P - (kk - s), P): disjoint and ascending since kk <= P
    const int pos = i < s ? i : P - kk + i;
    a.sel_pos[row + i] = pos;
    if (a.sel_slot) {
      const int page = a.page_table[(size_t)b * a.max_pages + pos / a.page_size];
      a.sel_slot[row + i] = page * a.page_size + pos % a.page_size;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.sel_count[b] = kk;
}

}  // namespace vg
