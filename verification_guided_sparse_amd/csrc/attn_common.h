// attn_common.h -- split-KV bookkeeping shared by the MFMA and VALU attention
// kernels: the per-workgroup merge of its waves' online-softmax states, the
// per-split partial results, and the combine of the splits of one
// (sequence, KV head).
//
// Every merge sums in a fixed order (wave 0..3, split 0..S-1), so results do
// not depend on which workgroup finishes first.
#pragma once

#include "vg_device.h"

namespace vg {

constexpr int kWaves = 4;           // waves per attention workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxRows = 64;        // rows (query rows x heads of a group) per workgroup

// LDS layout of the merge step.  O is staged as [wave][row][D] floats.
template <int ROWS, int D>
struct MergeSmem {
  float m[kWaves][ROWS];
  float l[kWaves][ROWS];
  float f[kWaves][ROWS];
  float o[kWaves][ROWS][D + 4];  // +4 floats per row: fewer LDS bank conflicts
};

// Step 1: each wave has written m[w][row] (log2 domain) and l[w][row] (full row
// sums).  Computes the per-wave weights f = exp2(m_w - max_w m_w) and writes
// this split's (m, l) for rows < M to part_ml.  Call between barriers.
template <int ROWS, int D>
__device__ __forceinline__ void merge_stats(MergeSmem<ROWS, D> &sm, float *part_ml, int M) {
  const int t = threadIdx.x;
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
    if (t < M) {
      part_ml[2 * t + 0] = mx;
      part_ml[2 * t + 1] = l;
    }
  }
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

__device__ __forceinline__ size_t part_index(const AttnArgs &a, int b, int g, int split) {
  return ((size_t)(b * a.num_kv_heads + g) * a.splits + split) * a.rows;
}

// Combine the splits of (b, g) for rows [row0, row0 + nrow) and write `out`.
// Thread `t` of `nt` handles a strided subset of (row, d).
template <int D>
__device__ __forceinline__ void combine_rows(const AttnArgs &a, int b, int g, int ns, int t, int nt) {
  const int M = a.rows, G = a.group_size;
  const float *pml = a.part_ml + part_index(a, b, g, 0) * 2;
  const float *po = a.part_o + part_index(a, b, g, 0) * D;
  for (int e = t * 4; e < M * D; e += nt * 4) {
    const int row = e / D, d = e % D;
    float mx = kMInit;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, pml[((size_t)s * M + row) * 2]);
    float den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
      const float f = exp2_fast(pml[((size_t)s * M + row) * 2] - mx);
      den += f * pml[((size_t)s * M + row) * 2 + 1];
      acc += f * *reinterpret_cast<const f32x4 *>(po + ((size_t)s * M + row) * D + d);
    }
    const float inv = 1.0f / den;
    const int r = row / G, h = g * G + row % G;
    *reinterpret_cast<f32x4 *>(a.out + (((size_t)b * a.nrows + r) * a.num_q_heads + h) * D + d) =
        acc * inv;
  }
}

// Separate combine launch: grid (ceil(M*D/(4*256)), Hkv, B), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  const int g = blockIdx.y, b = blockIdx.z;
  const SeqList s = seq_list(a, b);
  const int ns = num_splits_for(a, s.len);
  const int per_block = 4 * 256;
  // restrict this block to its slice of the M*D elements
  const int e0 = blockIdx.x * per_block;
  const int M = a.rows, G = a.group_size;
  const float *pml = a.part_ml + part_index(a, b, g, 0) * 2;
  const float *po = a.part_o + part_index(a, b, g, 0) * D;
  const int e = e0 + threadIdx.x * 4;
  if (e >= M * D) return;
  const int row = e / D, d = e % D;
  float mx = kMInit;
  for (int sp = 0; sp < ns; ++sp) mx = fmaxf(mx, pml[((size_t)sp * M + row) * 2]);
  float den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ns; ++sp) {
    const float f = exp2_fast(pml[((size_t)sp * M + row) * 2] - mx);
    den += f * pml[((size_t)sp * M + row) * 2 + 1];
    acc += f * *reinterpret_cast<const f32x4 *>(po + ((size_t)sp * M + row) * D + d);
  }
  const float inv = 1.0f / den;
  const int r = row / G, h = g * G + row % G;
  *reinterpret_cast<f32x4 *>(a.out + (((size_t)b * a.nrows + r) * a.num_q_heads + h) * D + d) =
      acc * inv;
}

// After a workgroup has written its partial: the last of the ns workgroups of
// (b, g) to finish combines all splits (counter reset to 0 for the next call).
template <int D>
__device__ __forceinline__ void finish_split(const AttnArgs &a, uint32_t *counters, int b, int g,
                                             int ns, int *sm_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t *c = counters + (b * a.num_kv_heads + g);
    const uint32_t ticket = atomicAdd(c, 1u);
    const int last = (ticket == (uint32_t)(ns - 1));
    if (last) atomicExch(c, 0u);
    *sm_flag = last;
  }
  __syncthreads();
  if (*sm_flag) {
    __threadfence();
    combine_rows<D>(a, b, g, ns, threadIdx.x, kThreads);
  }
}

}  // namespace vg
