// vg_device.h -- device-side types and helpers shared by the vegas_attn kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
// Running-max start value: finite, so exp2(m_old - m_new) stays 0 or 1 and never NaN.
constexpr float kMInit = -1.0e30f;
constexpr int kPageSize = 16;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Exponential in base 2 (hardware v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane 0's value of a float, as a wave-uniform value.  (readfirstlane takes
// an int: passing the float itself would convert its value, not its bits.)
__device__ __forceinline__ float first_lane(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Lane l exchanges with lane l ^ 32 / l ^ 16 through v_permlane32_swap /
// v_permlane16_swap: swapping a register with itself leaves {lower, upper}
// halves (resp. {even, odd} 16-lane rows) in the two results, so combining
// the two results gives the pairwise reduction in every lane.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum / max across the 4 sixteen-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_across_groups(float v) { return sum_xor32(sum_xor16(v)); }
__device__ __forceinline__ float max_across_groups(float v) { return max_xor32(max_xor16(v)); }

// DPP moves within a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum across the 16 lanes of a group (lanes sharing l / 16): pairs, quads,
// then the mirrored quad and the mirrored half-row.
__device__ __forceinline__ float sum_within_group(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}
// Inclusive prefix sum across the 64 lanes of a wave with DPP: shifts by
// 1, 2, 4, 8 inside each 16-lane row (lanes without a source read 0), then the
// last lane of row 0 (resp. of row 1) is broadcast into rows 1 and 3 (resp.
// rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive prefix sum over a 256-thread block (4 waves); `total` receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int *sm4, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) sm4[w] = x;
  __syncthreads();
  int pre = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = sm4[i];
    pre += (i < w) ? c : 0;
    total += c;
  }
  __syncthreads();
  return pre + x - v;
}

// Max across the 64 lanes without LDS: DPP inside each 16-lane row, then the
// lane swaps across rows.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  return max_across_groups(v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Arguments of one attention launch (verify or sparse draft).  The keys that
// (sequence b, KV head g) attends form a list of length L_b:
//   entries [0, cnt_b)    come from an explicit slot list (sparse: sel_slot),
//   entries [cnt_b, L_b)  are positions base_b + (i - cnt_b) translated through
//                         the page table (verify: the whole cache; sparse: the tail).
// Query row r (of nrows) sees entries i < L_b - nrows + 1 + r.
// Verify additionally exports the logits of rows 0 and gamma (or of every row)
// for entries i < P_b.
struct AttnArgs {
  const void *q;            // [B][nrows][Hq][D]
  const void *k_cache;      // [slots][Hkv][D]
  const void *v_cache;      // [slots][Hkv][D]
  const int32_t *page_table;  // [B][max_pages]
  const int32_t *sel_slot;    // [B][max_k] (sparse) or null
  const int32_t *sel_count;   // [B] (sparse) or null
  const int32_t *prefix_len;  // [B] (verify) or null
  const int32_t *tail_start;  // [B] (sparse) or null
  const int32_t *tail_len;    // [B] (sparse) or null
  float *out;               // [B][nrows][Hq][D]
  float *logits;            // [B][2][Hq][max_prefix] (all rows: [B][nrows][Hq][max_prefix]) or null
  float *group;             // [B][Hkv][max_prefix] or null
  float *part_o;            // [parts][M][D], parts = workgroups + B * Hkv
  float *part_ml;           // [parts][M][2]
  int32_t max_pages, max_k, max_prefix, max_tail;
  int32_t batch, nrows, gamma;
  int32_t num_q_heads, num_kv_heads, group_size, rows;  // rows = M = nrows * G
  int32_t workgroups;       // attention workgroups (grid size)
  int32_t tile;             // entries per tile of the attention kernel
  int32_t split_tokens;     // > 0: fixed splits of this many entries (see attn_common.h)
  int32_t splits;           // splits per (sequence, KV head) when split_tokens > 0
  int32_t export_all;       // 0: rows 0 and gamma exported (Collect-2-Query); 1: every row
  float scale;       // logit = scale * q.k (natural-log units)
  float scale_log2;  // scale * log2(e)
  int32_t sparse;
};

struct SeqList {
  int cnt, base, len, vis0, p_export;
};

__device__ __forceinline__ SeqList seq_list(const AttnArgs &a, int b) {
  SeqList s;
  if (a.sparse) {
    // counts clamped to the list and tail capacities the launch was sized for
    s.cnt = min(max(a.sel_count[b], 0), a.max_k);
    s.base = a.tail_start[b];
    s.len = s.cnt + min(max(a.tail_len[b], 1), a.max_tail);
    s.p_export = 0;
  } else {
    s.cnt = 0;
    s.base = 0;
    s.p_export = a.prefix_len[b];
    s.len = s.p_export + a.nrows;
  }
  s.vis0 = s.len - a.nrows + 1;
  return s;
}

// Physical slot of list entry i (0 <= i < len).
__device__ __forceinline__ int32_t entry_slot(const AttnArgs &a, int b, const SeqList &s, int i) {
  if (i < s.cnt) return a.sel_slot[(size_t)b * a.max_k + i];
  int pos = s.base + (i - s.cnt);
  return a.page_table[(size_t)b * a.max_pages + (pos >> 4)] * kPageSize + (pos & (kPageSize - 1));
}

// Work decomposition shared by the attention and combine kernels, for the key
// lists of the (sequence b, KV head g) segments, seg = b * Hkv + g:
//  * shared tiles (split_tokens == 0): the lists are cut in tiles and
//    concatenated; workgroup w of W takes tiles [w * T / W, (w + 1) * T / W) of
//    the T in total, whatever the sequence lengths (stream-K).  A workgroup's
//    share of one segment yields one partial result at index w + seg: along the
//    staircase of (w, seg) pairs each step raises w, seg or both, so these
//    indices are distinct and below W + B * Hkv.  Finding the shares needs the
//    lengths of all lists (one dependent load before any other).
//  * fixed splits (split_tokens > 0): workgroup w = seg * splits + sp takes
//    entries [sp * split_tokens, (sp + 1) * split_tokens) of its segment's list
//    and writes partial w, an empty one if the list is shorter.  Nothing
//    depends on the lengths, which suits short, latency-bound lists.
constexpr int kMaxBatch = 1024;

// Verify: the prefix length of sequence min(threadIdx.x, B - 1), loaded
// ahead of load_tile_prefix so that other loads can be in flight with it
// (unconditional and in bounds; the row count is added at use, so that
// nothing waits for the load here).
__device__ __forceinline__ int first_prefix_len(const AttnArgs &a) {
  return a.prefix_len[min((int)threadIdx.x, a.batch - 1)];
}

// pre[b] = sum over b' < b of ceil(len_b' / tile), for b <= B, and, if `lens`
// is given, lens[b] = len_b (LDS, all threads).  Returns (to all threads)
// whether every list has length `uniform_len`.  Verify callers may pass
// first_prefix_len(a) as p0 (have_p0) for sequences 0..255.
__device__ __forceinline__ bool load_tile_prefix(const AttnArgs &a, int *pre, int *sm4, int *lens = nullptr,
                                                 int uniform_len = -1, bool have_p0 = false, int p0 = 0) {
  int run = 0, differs = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 256) {
    const int b = b0 + (int)threadIdx.x;
    int len = 0;
    if (b < a.batch) len = (b0 == 0 && have_p0) ? p0 + a.nrows : seq_list(a, b).len;
    const int n = (len + a.tile - 1) / a.tile;
    if (lens && b < a.batch) lens[b] = len;
    differs |= (b < a.batch && len != uniform_len);
    int tot;
    const int ex = block_exclusive_scan(n, sm4, tot);
    if (b < a.batch) pre[b] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) pre[a.batch] = run;
  return !__syncthreads_or(differs);
}

// floor(num / den) for 0 <= num < 2^52 and 0 < den < 2^31: the double
// quotient is within one of it and is corrected by one step (a 64-bit integer
// division is a long software sequence on the GPU).
__host__ __device__ inline long long floor_div(long long num, long long den) {
  long long q = (long long)((double)num / (double)den);
  if (q * den > num)
    --q;
  else if ((q + 1) * den <= num)
    ++q;
  return q;
}

__host__ __device__ inline long long share_begin(int w, long long T, int W) {
  return floor_div((long long)w * T, W);
}

}  // namespace vg
