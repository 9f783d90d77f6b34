// attn_valu.h -- attention over paged key lists with the contraction on the vector ALUs
// (fp32 FMA).  Serves fp32 caches and is the comparison point for the MFMA
// kernel on bf16.  Same key lists, masking, export and work sharing as
// attn_mfma.h.
//
// Workgroups share the 64-entry tiles of all key lists (attn_common.h); for
// each piece of its share a workgroup stages the M query rows of KV head g in
// LDS as fp32, and each wave walks the piece's tiles t = wave, wave + 4, ...:
//   QK: lane <-> key entry; the lane streams its key row and forms all M dot
//       products against LDS-broadcast query rows;
//   softmax: per row across the wave (shuffle reductions);
//   PV: lane <-> DV = D/64 output columns; V rows are read coalesced, the
//       probabilities come from LDS.
#pragma once

#include "attn_common.h"

namespace vg {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static void load16(const void *p, float *out) {
    const f32x4 v = __builtin_nontemporal_load(static_cast<const f32x4 *>(p));
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
  __device__ static float load1(const void *p, size_t i) { return static_cast<const float *>(p)[i]; }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
  __device__ static void load16(const void *p, float *out) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ static float load1(const void *p, size_t i) {
    return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
  }
};

template <int MR, int D>
struct ValuSmem {
  union {
    struct {
      float q[MR][D];
      float p[kWaves][MR][kWave];
      int slot[kWaves][kWave];
    } loop;
    MergeSmem<MR, D> merge;
  };
};

template <typename T, int D, int MR>
__global__ __launch_bounds__(kThreads, 1) void attn_valu_kernel(AttnArgs a) {
  constexpr int DV = D / kWave;  // output columns per lane
  constexpr int CH = Elem<T>::kPer16B;
  __shared__ ValuSmem<MR, D> sm;
  __shared__ int pre[kMaxBatch + 1];
  __shared__ int lens[kMaxBatch];
  __shared__ int sm4[4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.group_size, M = a.rows, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const size_t slot_elems = (size_t)Hkv * D;
  const bool do_export = !a.sparse && (a.logits != nullptr || a.group != nullptr);

  for_each_piece(a, pre, lens, sm4, [&](int b, int g, int part, int e_begin, int e_end) {
    const SeqList s = seq_list(a, b);
    __syncthreads();  // the previous piece's merge has read the LDS
    for (int i = threadIdx.x; i < MR * D; i += kThreads) {
      const int row = i / D, d = i % D;
      float v = 0.f;
      if (row < M) {
        const int r = row / G, h = g * G + row % G;
        v = Elem<T>::load1(a.q, ((size_t)(b * a.nrows + r) * Hq + h) * D + d);
      }
      sm.loop.q[row][d] = v;
    }
    __syncthreads();

    float o[MR][DV];
    float m_run[MR], l_run[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      m_run[m] = kMInit;
      l_run[m] = 0.f;
#pragma unroll
      for (int k = 0; k < DV; ++k) o[m][k] = 0.f;
    }

    const int ntiles = (e_end - e_begin + kWave - 1) / kWave;
    for (int t = wave; t < ntiles; t += kWaves) {
      const int e0 = e_begin + t * kWave;
      const int e = e0 + lane;
      const int slot = entry_slot(a, b, s, min(e, e_end - 1));
      sm.loop.slot[wave][lane] = slot;

      float acc[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = 0.f;
      const T *krow = static_cast<const T *>(a.k_cache) + (size_t)slot * slot_elems + (size_t)g * D;
      for (int d0 = 0; d0 < D; d0 += CH) {
        float kv[CH];
        Elem<T>::load16(krow + d0, kv);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          float sacc = 0.f;
#pragma unroll
          for (int c = 0; c < CH; ++c) sacc = fmaf(sm.loop.q[m][d0 + c], kv[c], sacc);
          acc[m] += sacc;
        }
      }

      if (do_export && e0 < s.p_export) {
        float gs = 0.f;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const int r = m / G, h = g * G + m % G;
            const float l = acc[m] * a.scale;
            if (e < s.p_export) {
              if (a.logits && r == 0) a.logits[((size_t)(b * 2 + 0) * Hq + h) * a.max_prefix + e] = l;
              if (a.logits && r == a.gamma) a.logits[((size_t)(b * 2 + 1) * Hq + h) * a.max_prefix + e] = l;
            }
            gs += (float)((r == 0) + (r == a.gamma)) * acc[m];
          }
        }
        if (a.group && e < s.p_export) a.group[(size_t)(b * Hkv + g) * a.max_prefix + e] = gs * a.scale;
      }

      float alpha[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int vis = s.vis0 + m / G;
        const bool ok = (e < e_end) && (e < vis);
        const float x = ok ? acc[m] * a.scale_log2 : kNegInf;
        const float m_new = fmaxf(m_run[m], wave_max(x));
        alpha[m] = exp2_fast(m_run[m] - m_new);
        m_run[m] = m_new;
        const float p = exp2_fast(x - m_new);
        l_run[m] = l_run[m] * alpha[m] + p;
        sm.loop.p[wave][m][lane] = p;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int k = 0; k < DV; ++k) o[m][k] *= alpha[m];
      const int jn = min(kWave, e_end - e0);
      for (int j = 0; j < jn; ++j) {
        const int sj = sm.loop.slot[wave][j];
        const T *vrow = static_cast<const T *>(a.v_cache) + (size_t)sj * slot_elems + (size_t)g * D;
        float vv[DV];
#pragma unroll
        for (int k = 0; k < DV; ++k) vv[k] = Elem<T>::load1(vrow, lane * DV + k);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const float p = sm.loop.p[wave][m][j];
#pragma unroll
          for (int k = 0; k < DV; ++k) o[m][k] = fmaf(p, vv[k], o[m][k]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }

    __syncthreads();  // the merge area aliases the loop buffers
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float lsum = wave_sum(l_run[m]);
      if (lane == 0) {
        sm.merge.m[wave][m] = m_run[m];
        sm.merge.l[wave][m] = lsum;
      }
    }
    __syncthreads();
    const size_t pidx = (size_t)part * M;
    const RowStat st = merge_stats<MR, D>(sm.merge);
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int k = 0; k < DV; ++k) sm.merge.o[wave][m][lane * DV + k] = o[m][k];
    __syncthreads();
    merge_o<MR, D>(sm.merge, a.part_o + pidx * D, M);
    store_stats(a.part_ml + pidx * 2, M, st);
  });
}

}  // namespace vg
