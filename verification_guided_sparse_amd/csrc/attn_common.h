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

// Combining the splits of (b, g): out = sum_s w_s O_s / sum_s w_s l_s with
// w_s = exp2(m_s - max_s m_s), for rows [row0, row0 + nr).  The loads of each
// phase are independent of one another, so they are in flight together rather
// than forming a chain of dependent loads.
//
// LDS: `wsm` holds 2 * ns * nr + 2 * nr floats, `acc_sm` 4 * 256 floats.
constexpr int kMaxSplits = 512;

template <int D>
__device__ __forceinline__ void combine_rows(const AttnArgs &a, int b, int g, int ns, int row0,
                                             int nr, float *wsm, float *acc_sm) {
  constexpr int C = D / 4;  // float4 columns of a row
  const int M = a.rows, G = a.group_size, t = threadIdx.x;
  const float *pml = a.part_ml + part_index(a, b, g, 0) * 2;
  const float *po = a.part_o + part_index(a, b, g, 0) * D;
  const int n = ns * nr;
  float *wm = wsm, *wl = wsm + n, *mx = wsm + 2 * n, *den = mx + nr;
  // 1. every split's (m, l) of every row
  for (int i = t; i < n; i += kThreads) {
    const int sp = i / nr, r = i % nr;
    const float *e = pml + ((size_t)sp * M + row0 + r) * 2;
    wm[i] = e[0];
    wl[i] = e[1];
  }
  __syncthreads();
  for (int r = t; r < nr; r += kThreads) {
    float m = kMInit;
    for (int sp = 0; sp < ns; ++sp) m = fmaxf(m, wm[sp * nr + r]);
    mx[r] = m;
  }
  __syncthreads();
  // 2. split weights and denominators
  for (int i = t; i < n; i += kThreads) {
    const float w = exp2_fast(wm[i] - mx[i % nr]);
    wm[i] = w;
    wl[i] *= w;
  }
  __syncthreads();
  for (int r = t; r < nr; r += kThreads) {
    float d = 0.f;
    for (int sp = 0; sp < ns; ++sp) d += wl[sp * nr + r];
    den[r] = d;
  }
  __syncthreads();
  // 3. weighted sum of the partial outputs: (row, column) pairs x split groups
  const int tc = nr * C;
  const int sp_par = tc >= kThreads ? 1 : kThreads / tc;
  const size_t stride = (size_t)M * D;
  for (int base = 0; base < tc; base += kThreads) {
    const int idx = (sp_par > 1) ? (t % tc) : (base + t);
    const int sg = (sp_par > 1) ? (t / tc) : 0;
    const bool active = (sp_par > 1) ? (t < sp_par * tc) : (idx < tc);
    const int r = idx / C, col = idx % C;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      const float *src = po + (size_t)(row0 + r) * D + 4 * col;
      int sp = sg;
      for (; sp + 3 * sp_par < ns; sp += 4 * sp_par) {
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(src + (size_t)sp * stride);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(src + (size_t)(sp + sp_par) * stride);
        const f32x4 v2 = *reinterpret_cast<const f32x4 *>(src + (size_t)(sp + 2 * sp_par) * stride);
        const f32x4 v3 = *reinterpret_cast<const f32x4 *>(src + (size_t)(sp + 3 * sp_par) * stride);
        acc += wm[sp * nr + r] * v0;
        acc += wm[(sp + sp_par) * nr + r] * v1;
        acc += wm[(sp + 2 * sp_par) * nr + r] * v2;
        acc += wm[(sp + 3 * sp_par) * nr + r] * v3;
      }
      for (; sp < ns; sp += sp_par)
        acc += wm[sp * nr + r] * *reinterpret_cast<const f32x4 *>(src + (size_t)sp * stride);
    }
    bool write = active;
    if (sp_par > 1) {
      *reinterpret_cast<f32x4 *>(acc_sm + 4 * t) = acc;
      __syncthreads();
      write = t < tc;
      if (write) {
        for (int j = 1; j < sp_par; ++j)
          acc += *reinterpret_cast<const f32x4 *>(acc_sm + 4 * (j * tc + t));
      }
    }
    if (write) {
      const int row = row0 + r;
      const int qr = row / G, h = g * G + row % G;
      *reinterpret_cast<f32x4 *>(a.out + (((size_t)b * a.nrows + qr) * a.num_q_heads + h) * D + 4 * col) =
          acc * (1.0f / den[r]);
    }
    __syncthreads();
  }
}

// Separate combine launch: one block per (row, g, b), 256 threads.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(AttnArgs a) {
  __shared__ float wsm[2 * kMaxSplits + 2];
  __shared__ float acc_sm[kThreads * 4];
  const int row = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const SeqList s = seq_list(a, b);
  const int ns = num_splits_for(a, s.len);
  combine_rows<D>(a, b, g, ns, row, 1, wsm, acc_sm);
}

// After a workgroup has written its partial: the last of the ns workgroups of
// (b, g) to finish combines all splits (counter reset to 0 for the next call).
// `scratch` is dead LDS of at least 4 * 256 + 2 * (ns + 1) * M floats.
template <int D>
__device__ __forceinline__ void finish_split(const AttnArgs &a, uint32_t *counters, int b, int g,
                                             int ns, int *sm_flag, float *scratch) {
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
    combine_rows<D>(a, b, g, ns, 0, a.rows, scratch + kThreads * 4, scratch);
  }
}

}  // namespace vg
