// kv_append.h -- writing the new tokens' K/V rows into the paged cache: the
// step that precedes verification (the gamma+1 tokens of an iteration must be
// in the cache before verify attends to them), done here so that a whole
// iteration can stay on the device.
//
// One workgroup per (token r, sequence b) moves the token's Hkv * D elements
// of K and of V as 16-byte vectors: reads and writes are fully coalesced, and
// the kernel is bound by HBM bandwidth (2 x 2 x Hkv * D * elem bytes per token).
#pragma once

#include "vg_device.h"

namespace vg {

struct AppendArgs {
  const void *k_new, *v_new;  // [B][n_new][Hkv][D]
  void *k_cache, *v_cache;    // [num_slots][Hkv][D]
  const int32_t *page_table;  // [B][max_pages]
  const int32_t *start_pos;   // [B]: logical position of new token 0
  int32_t n_new, max_pages, row_vec16;  // row_vec16: 16-byte vectors per token (Hkv * D * elem / 16)
};

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int r = blockIdx.x, b = blockIdx.y;
  const int pos = a.start_pos[b] + r;
  const int page_idx = pos >> 4;
  // positions outside the sequence's page-table row are skipped (precondition
  // violations are not turned into out-of-bounds writes)
  if (pos < 0 || page_idx >= a.max_pages) return;
  const int page = a.page_table[(size_t)b * a.max_pages + page_idx];
  if (page < 0) return;
  const size_t slot = (size_t)page * kPageSize + (pos & (kPageSize - 1));
  const size_t src = ((size_t)b * a.n_new + r) * a.row_vec16;
  const u32x4 *ks = static_cast<const u32x4 *>(a.k_new) + src;
  const u32x4 *vs = static_cast<const u32x4 *>(a.v_new) + src;
  u32x4 *kd = static_cast<u32x4 *>(a.k_cache) + slot * a.row_vec16;
  u32x4 *vd = static_cast<u32x4 *>(a.v_cache) + slot * a.row_vec16;
  for (int i = threadIdx.x; i < a.row_vec16; i += blockDim.x) {
    const u32x4 kv = __builtin_nontemporal_load(ks + i);
    const u32x4 vv = __builtin_nontemporal_load(vs + i);
    kd[i] = kv;
    vd[i] = vv;
  }
}

// Keeping the accepted tokens: prefix_len[b] += 1 + clamp(n_accepted[b], 0, gamma).
// One thread per sequence; the next append then starts at the new prefix end.
__global__ __launch_bounds__(256) void advance_prefix_kernel(int32_t batch, int32_t gamma,
                                                           const int32_t *n_accepted, int32_t *prefix_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  prefix_len[b] += 1 + min(max(n_accepted[b], 0), gamma);
}

}  // namespace vg
