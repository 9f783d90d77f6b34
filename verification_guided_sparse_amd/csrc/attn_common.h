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

// Combining the splits of (b, g) for one output row:
//   out = sum_s w_s O_s / sum_s w_s l_s,  w_s = exp2(m_s - max_s m_s).
// One 256-thread block per row; thread (split group sg, float4 column col)
// takes splits sg, sg + SP, ... in batches of kBatch whose (m, l, O) loads are
// all in flight together, keeping an online (max, denominator, sum) state; the
// groups' states are then merged through LDS.  One batch covers
// kBatch * SP >= 64 splits, so a typical row costs one memory round trip.
constexpr int kMaxSplits = 512;

template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(AttnArgs a) {
  constexpr int C = D / 4;          // float4 columns of a row
  constexpr int SP = kThreads / C;  // split groups
  constexpr int kBatch = 8;
  __shared__ float sm_m[kThreads];
  __shared__ float sm_d[SP];
  __shared__ f32x4 sm_o[kThreads];
  const int row = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const SeqList s = seq_list(a, b);
  const int ns = num_splits_for(a, s.len);
  const int M = a.rows, G = a.group_size;
  const int col = t % C, sg = t / C;
  const float *pml = a.part_ml + (part_index(a, b, g, 0) + row) * 2;
  const float *po = a.part_o + (part_index(a, b, g, 0) + row) * D + 4 * col;
  const size_t ml_stride = (size_t)M * 2, o_stride = (size_t)M * D;

  float mt = kMInit, dt = 0.f;
  f32x4 at = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < ns; s0 += kBatch * SP) {
    float m[kBatch], l[kBatch];
    f32x4 o[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int sp = s0 + i * SP;
      const bool ok = sp < ns;
      m[i] = ok ? pml[sp * ml_stride] : kMInit;
      l[i] = ok ? pml[sp * ml_stride + 1] : 0.f;
      o[i] = ok ? *reinterpret_cast<const f32x4 *>(po + sp * o_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
  }
  // merge the split groups: max, then rescaled sums
  sm_m[t] = mt;
  __syncthreads();
  float mx = kMInit;
  for (int j = 0; j < SP; ++j) mx = fmaxf(mx, sm_m[j * C + col]);
  const float r = exp2_fast(mt - mx);
  sm_o[t] = at * r;
  if (col == 0) sm_d[sg] = dt * r;
  __syncthreads();
  if (t < C) {
    f32x4 acc = sm_o[t];
    float den = sm_d[0];
    for (int j = 1; j < SP; ++j) {
      acc += sm_o[j * C + t];
      den += sm_d[j];
    }
    const int qr = row / G, h = g * G + row % G;
    *reinterpret_cast<f32x4 *>(a.out + (((size_t)b * a.nrows + qr) * a.num_q_heads + h) * D + 4 * t) =
        acc * (1.0f / den);
  }
}

}  // namespace vg
