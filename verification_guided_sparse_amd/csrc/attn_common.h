// attn_common.h -- work sharing bookkeeping of the MFMA and VALU attention
// kernels: the walk over a workgroup's share of the key tiles, the merge of its
// waves' online-softmax states into one partial result per piece, and the
// combine of the partials of one (sequence, KV head).
//
// Every merge sums in a fixed order (wave 0..3, workgroups in index order), so
// results do not depend on which workgroup finishes first.
#pragma once

#include "vg_device.h"

namespace vg {

constexpr int kWaves = 4;           // waves per attention workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxRows = 64;        // rows (query rows x heads of a group) per workgroup

// PF = tiles in flight per wave.  PF == 1: load, then compute, two waves per
// SIMD; PF > 1: a ring of PF tiles, one wave per SIMD.
// SPARSE selects the sparse draft (true) or verify (false) instantiation; the
// local copy of the arguments carries it as a constant, so every helper that
// tests a.sparse folds to one path.
// Workgroups per CU the kernel is compiled for.  The sparse draft takes two
// where its rows fit the registers of two (at D = 128 with 2 row tiles they
// would spill).  Verify at D = 64 with at most
// 3 row tiles fits two workgroups (one tile in flight per wave): the second
// workgroup's waves hide the first's softmax work, which per byte is twice
// that of D = 128.  D = 128 verify keeps one workgroup with two tiles in
// flight (at two it spills and is slower).
constexpr int attn_occupancy(int D, int NT, int PF, bool sparse) {
  return sparse ? ((PF == 1 && (NT == 1 || (D == 64 && NT == 2))) ? 2 : 1)
                : ((D == 64 && NT <= 3 && PF == 1) ? 2 : 1);
}

// LDS layout of the merge step.  O is staged as [wave][row][D] floats.
template <int ROWS, int D>
struct MergeSmem {
  float m[kWaves][ROWS];
  float l[kWaves][ROWS];
  float f[kWaves][ROWS];
  float o[kWaves][ROWS][D + 4];  // +4 floats per row: fewer LDS bank conflicts
};

// Step 1: each wave has written m[w][row] (log2 domain) and l[w][row] (full row
// sums).  Computes the per-wave weights f = exp2(m_w - max_w m_w) into LDS and
// returns this piece's (m, l) for row t = threadIdx.x (meaningful for t < M).
// Call between barriers.  The caller stores the pair with store_stats after
// merge_o: a global store here would make the O writes that follow wait for it
// (the registers it reads are reused), a full memory round trip.
struct RowStat {
  float m, l;
};

template <int ROWS, int D>
__device__ __forceinline__ RowStat merge_stats(MergeSmem<ROWS, D> &sm) {
  const int t = threadIdx.x;
  RowStat r{kMInit, 0.f};
  if (t < ROWS) {
    float mx = sm.m[0][t];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][t]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      float f = exp2_fast(sm.m[w][t] - mx);
      sm.f[w][t] = f;
      l += f * sm.l[w][t];
    }
    r.m = mx;
    r.l = l;
  }
  return r;
}

__device__ __forceinline__ void store_stats(float *part_ml, int M, RowStat r) {
  const int t = threadIdx.x;
  if (t < M) *reinterpret_cast<f32x2 *>(part_ml + 2 * t) = f32x2{r.m, r.l};
}

// Step 2: each wave has written its O (unscaled) to sm.o[w].  Writes the
// weighted sum over waves for rows < M to part_o ([M][D]).
template <int ROWS, int D>
__device__ __forceinline__ void merge_o(MergeSmem<ROWS, D> &sm, float *part_o, int M) {
  for (int e = threadIdx.x * 4; e < M * D; e += kThreads * 4) {
    const int row = e / D, d = e % D;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = sm.f[w][row];
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&sm.o[w][row][d]);
      acc += f * v;
    }
    *reinterpret_cast<f32x4 *>(part_o + e) = acc;
  }
}

// ---- work split index math (host and device; the host build is tested) ----

// Stream-K walk of workgroup w: tiles [t, t_end) remain, the next one in
// sequence b.  pre[b] = tiles of sequences before b (pre[batch] = all): an
// array, or UniformPre when every list has the same number of tiles.
struct ShareWalk {
  int t, t_end, b;
};

struct UniformPre {
  int n;  // tiles of every list
  __host__ __device__ int operator[](int b) const { return b * n; }
};

template <typename Pre>
__host__ __device__ inline ShareWalk share_walk_begin(const Pre &pre, int batch, int Hkv, int w, int W) {
  ShareWalk s;
  const long long T = (long long)Hkv * pre[batch];
  s.t = (int)share_begin(w, T, W);
  s.t_end = (int)share_begin(w + 1, T, W);
  // sequence holding tile t: largest b with Hkv * pre[b] <= t
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)Hkv * pre[mid] <= s.t) lo = mid; else hi = mid - 1;
  }
  s.b = lo;
  return s;
}

// A piece: entries [e_begin, e_end) of the list of sequence b, KV head g,
// whose partial result goes to index `part`.
struct Piece {
  int b, g, part, e_begin, e_end;
};

// Next piece of a stream-K walk (call while s.t < s.t_end); len[b] = list lengths.
template <typename Pre, typename LenFn>
__host__ __device__ inline Piece share_walk_next(ShareWalk &s, const Pre &pre, int Hkv, int tile, int w,
                                                 LenFn len) {
  int n = pre[s.b + 1] - pre[s.b];
  while (n == 0) {  // lists without tiles (none for valid inputs)
    ++s.b;
    n = pre[s.b + 1] - pre[s.b];
  }
  const int sb = Hkv * pre[s.b];
  Piece p;
  p.b = s.b;
  p.g = (s.t - sb) / n;
  const int seg_start = sb + p.g * n;
  const int hi_t = s.t_end < seg_start + n ? s.t_end : seg_start + n;
  const int L = len(p.b);
  p.e_begin = (s.t - seg_start) * tile;
  p.e_end = (hi_t - seg_start) * tile;
  if (p.e_end > L) p.e_end = L;
  p.part = w + p.b * Hkv + p.g;
  s.t = hi_t;
  if (p.g == Hkv - 1 && s.t == seg_start + n) ++s.b;  // the next piece starts in the next sequence
  return p;
}

// The piece of workgroup w with fixed splits (empty past the list's end).
__host__ __device__ inline Piece fixed_piece(int w, int splits, int split_tokens, int Hkv, int list_len) {
  Piece p;
  const int seg = w / splits, sp = w % splits;
  p.b = seg / Hkv;
  p.g = seg % Hkv;
  p.part = w;
  const long long e0 = (long long)sp * split_tokens;
  p.e_begin = (int)(e0 < list_len ? e0 : list_len);
  p.e_end = (int)(e0 + split_tokens < list_len ? e0 + split_tokens : list_len);
  return p;
}

// Partials of segment (b, g) for the combine: indices first + j, j < count.
// With shared tiles, index first + j is only valid if workgroup w = first + j -
// seg has a share that meets the segment (share_meets).
template <typename Pre>
__host__ __device__ inline void combine_range(const Pre &pre, int batch, int Hkv, int W, int b, int g,
                                              int &first, int &count) {
  const long long T = (long long)Hkv * pre[batch];
  const int n = pre[b + 1] - pre[b];
  const long long S = (long long)Hkv * pre[b] + (long long)g * n;  // segment's first tile
  // workgroups whose share [share_begin(w), share_begin(w + 1)) meets [S, S + n)
  int w_first = (int)floor_div((S + 1) * W + T - 1, T) - 1;
  int w_last = (int)floor_div((S + n) * W + T - 1, T) - 1;
  w_first = w_first < 0 ? 0 : (w_first > W - 1 ? W - 1 : w_first);
  w_last = w_last > W - 1 ? W - 1 : w_last;
  if (w_last < w_first) w_last = w_first;
  first = w_first + b * Hkv + g;
  count = w_last - w_first + 1;
}

template <typename Pre>
__host__ __device__ inline bool share_meets(const Pre &pre, int batch, int Hkv, int W, int w, int b, int g) {
  const long long T = (long long)Hkv * pre[batch];
  const int n = pre[b + 1] - pre[b];
  const long long S = (long long)Hkv * pre[b] + (long long)g * n;
  const long long lo = share_begin(w, T, W), hi = share_begin(w + 1, T, W);
  return (lo > S ? lo : S) < (hi < S + n ? hi : S + n);
}

// Combining the partials of segment (b, g) for one output row:
//   out = sum_w c_w O_w / sum_w c_w l_w,  c_w = exp2(m_w - max_w m_w)
// over the workgroups w whose share of the tiles meets the segment (or over
// the segment's fixed splits).  RPB rows per 256-thread block (fewer blocks
// when each row has few partials: many tiny blocks are limited by how fast
// they are dispatched); thread (group sg, float4 column col) of a row takes
// partials sg, sg + SP, ... in batches whose (m, l, O) loads are all in
// flight together, keeping an online (max, denominator, sum) state; the
// groups' states are then merged through LDS.
template <int D, int RPB>
__device__ __forceinline__ void combine_block(const AttnArgs &a, int bx, int g, int b) {
  constexpr int C = D / 4;              // float4 columns of a row
  constexpr int TPR = kThreads / RPB;   // threads per row
  constexpr int SP = TPR / C;           // partial groups per row
  static_assert(SP >= 1, "a row needs at least one partial group");
  constexpr int kBatch = 8;
  __shared__ int pre[kMaxBatch + 1];
  __shared__ int sm4[4];
  __shared__ float sm_m[kThreads];
  __shared__ float sm_d[RPB * SP];
  __shared__ f32x4 sm_o[kThreads];
  const int t = threadIdx.x;
  const int rg = t / TPR, tr = t % TPR;  // this thread's row in the block, its index in the row
  const int row = bx * RPB + rg;
  const int Hkv = a.num_kv_heads, W = a.workgroups;
  const bool fixed = a.split_tokens > 0;
  const int seg = b * Hkv + g, M = a.rows;
  const bool live = row < M;  // the last block may hold fewer rows (no early exit: barriers)
  const int col = tr % C, sg = tr / C;
  const size_t ml_stride = (size_t)M * 2, o_stride = (size_t)M * D;
  float mt = kMInit, dt = 0.f;
  f32x4 at = {0.f, 0.f, 0.f, 0.f};
  float m[kBatch], l[kBatch];
  f32x4 o[kBatch];
  // Merges a batch into the running (max, denominator, sum).
  auto accumulate = [&]() {
    float mb = mt;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) mb = fmaxf(mb, m[i]);
    const float r = exp2_fast(mt - mb);
    dt *= r;
    at *= r;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = exp2_fast(m[i] - mb);
      dt += w * l[i];
      at += w * o[i];
    }
    mt = mb;
  };
  // Batch j0, j0 + SP, ... of the partials of range [first, first + np)
  // (partial j at (first + j) * M + row); those failing ok(partial index)
  // count as empty.
  auto load_batch = [&](int first, int np, int j0, auto ok_fn) {
    const size_t p0 = (size_t)first * M + row;
    const float *pml = a.part_ml + p0 * 2;
    const float *po = a.part_o + p0 * D + 4 * col;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = j0 + i * SP;
      const bool ok = live && j < np && ok_fn(first + j);
      m[i] = ok ? pml[j * ml_stride] : kMInit;
      l[i] = ok ? pml[j * ml_stride + 1] : 0.f;
      o[i] = ok ? *reinterpret_cast<const f32x4 *>(po + j * o_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto all = [](int) { return true; };

  if (fixed) {  // partials seg * splits .. + splits - 1, all written
    const int first = seg * a.splits, np = a.splits;
    for (int j0 = sg; j0 < np; j0 += kBatch * SP) {
      load_batch(first, np, j0, all);
      accumulate();
    }
  } else {
    // Shared tiles (verify lists).  Partial p of a segment's range is written
    // if workgroup p - seg has a share that meets the segment, which holds for
    // the whole range when every workgroup has tiles (W <= T).
    //
    // Speculation: with every list at its longest length (all prefixes equal
    // to max_prefix) the range is known before the lengths are read, so its
    // first batch is loaded together with them (issued unconditionally, a
    // partial outside the range reading partial 0 of the range instead, and
    // masked after) and kept if the lengths agree.
    const int spec_len = a.max_prefix + a.nrows;
    const UniformPre up{(spec_len + a.tile - 1) / a.tile};
    const int p0 = first_prefix_len(a);  // in flight with the speculative loads
    int first, np;
    combine_range(up, a.batch, Hkv, W, b, g, first, np);
    const bool up_all = W <= (long long)Hkv * up[a.batch];
    {
      const size_t q0 = (size_t)first * M + (live ? row : 0);
      const float *pml = a.part_ml + q0 * 2;
      const float *po = a.part_o + q0 * D + 4 * col;
      bool ok[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int j = sg + i * SP;
        ok[i] = live && j < np && (up_all || share_meets(up, a.batch, Hkv, W, first + j - seg, b, g));
        const int jj = ok[i] ? j : 0;
        const f32x2 ml = *reinterpret_cast<const f32x2 *>(pml + jj * ml_stride);
        m[i] = ml[0];
        l[i] = ml[1];
        o[i] = *reinterpret_cast<const f32x4 *>(po + jj * o_stride);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (!ok[i]) {
          m[i] = kMInit;
          l[i] = 0.f;
          o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    const bool spec = load_tile_prefix(a, pre, sm4, nullptr, spec_len, true, p0);
    if (!spec) combine_range(pre, a.batch, Hkv, W, b, g, first, np);
    const bool every = W <= (long long)Hkv * pre[a.batch];
    auto meets = [&](int p) { return share_meets(pre, a.batch, Hkv, W, p - seg, b, g); };
    for (int j0 = sg; j0 < np; j0 += kBatch * SP) {
      if (j0 != sg || !spec) {
        if (every)
          load_batch(first, np, j0, all);
        else
          load_batch(first, np, j0, meets);
      }
      accumulate();
    }
  }
  const int G = a.group_size;

  // merge each row's groups: max, then rescaled sums
  const int rb = rg * TPR;  // this row's threads in the block
  sm_m[t] = mt;
  __syncthreads();
  float mx = kMInit;
  for (int j = 0; j < SP; ++j) mx = fmaxf(mx, sm_m[rb + j * C + col]);
  const float r = exp2_fast(mt - mx);
  sm_o[t] = at * r;
  if (col == 0) sm_d[rg * SP + sg] = dt * r;
  __syncthreads();
  if (live && tr < C) {
    f32x4 acc = sm_o[rb + tr];
    float den = sm_d[rg * SP];
    for (int j = 1; j < SP; ++j) {
      acc += sm_o[rb + j * C + tr];
      den += sm_d[rg * SP + j];
    }
    const int qr = row / G, h = g * G + row % G;
    *reinterpret_cast<f32x4 *>(a.out + (((size_t)b * a.nrows + qr) * a.num_q_heads + h) * D + 4 * tr) =
        acc * (1.0f / den);
  }
}

// Combine blocks of one or more rows per (KV head, sequence): grid
// (ceil(M / RPB), Hkv, B).
template <int D, int RPB>
__global__ __launch_bounds__(kThreads) void combine_kernel(AttnArgs a) {
  combine_block<D, RPB>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// x of the first active lane (a wave-uniform value the compiler may keep in a
// scalar register).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Calls fn(b, g, part, e_begin, e_end) for each piece of this workgroup's work
// (uniform across the block): entries [e_begin, e_end) of the list of segment
// (b, g), whose partial result goes to index `part`.  With fixed splits a
// workgroup past its list's end gets one empty piece (e_begin == e_end).
// pre / lens / sm4: LDS for load_tile_prefix.
template <typename Fn>
__device__ __forceinline__ void for_each_piece(const AttnArgs &a, int *pre, int *lens, int *sm4, Fn fn) {
  const int W = a.workgroups, w = blockIdx.x, Hkv = a.num_kv_heads;
  const bool fixed = a.split_tokens > 0;
  ShareWalk s{0, 1, 0};
  if (!fixed) {
    load_tile_prefix(a, pre, sm4, lens);  // lists' lengths kept in LDS: no second load
    s = share_walk_begin(pre, a.batch, Hkv, w, W);
  }
  auto len = [&](int b) { return fixed ? seq_list(a, b).len : lens[b]; };
  // One call site for fn, so that it is inlined once.
  while (s.t < s.t_end) {
    Piece p;
    if (fixed) {
      const int b = w / a.splits / Hkv;
      p = fixed_piece(w, a.splits, a.split_tokens, Hkv, len(b));
      s.t = s.t_end;
    } else {
      p = share_walk_next(s, pre, Hkv, a.tile, w, len);
    }
    // wave-uniform values: scalar registers
    fn(uniform(p.b), uniform(p.g), uniform(p.part), uniform(p.e_begin), uniform(p.e_end));
  }
}

}  // namespace vg
