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
  __device__ static float load1(const void *p, size_t i) { return static_cast<const float *>(p)[i]; }
  __device__ static void convert16(const u32x4 &v, float *out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
  __device__ static float load1(const void *p, size_t i) {
    return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
  }
  __device__ static void convert16(const u32x4 &v, float *out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};

template <int MR, int D>
struct ValuSmem {
  union {
    struct {
      float q[MR][D];
      float p[kWaves][MR][kWave];
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
    constexpr int NK = D / CH;  // 16-byte chunks of a K row
    const T *kbase = static_cast<const T *>(a.k_cache) + (size_t)g * D;
    const T *vbase = static_cast<const T *>(a.v_cache) + (size_t)g * D + lane * DV;
    for (int t = wave; t < ntiles; t += kWaves) {
      const int e0 = e_begin + t * kWave;
      const int e = e0 + lane;
      // entries past the end reuse the last one's slot; their p is 0
      const int slot = entry_slot(a, b, s, min(e, e_end - 1));
      // This lane's K row, all chunks in flight together.
      u32x4 kraw[NK];
      const T *krow = kbase + (size_t)slot * slot_elems;
#pragma unroll
      for (int c = 0; c < NK; ++c) kraw[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(krow + c * CH));

      float acc[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        float kv[CH];
        Elem<T>::convert16(kraw[c], kv);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
#pragma unroll
          for (int c4 = 0; c4 < CH; c4 += 4) {
            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&sm.loop.q[m][c * CH + c4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m] = fmaf(q4[i], kv[c4 + i], acc[m]);
          }
        }
      }

      // This lane's DV columns of the 64 V rows (entry j's slot comes from lane
      // j), issued after QK so that they do not hold registers through it;
      // they land during the export and softmax.
      float vv[kWave][DV];
#pragma unroll
      for (int j = 0; j < kWave; ++j) {
        const int sj = __builtin_amdgcn_readlane(slot, j);  // wave-uniform: scalar address
#pragma unroll
        for (int k = 0; k < DV; ++k) vv[j][k] = Elem<T>::load1(vbase + (size_t)sj * slot_elems, k);
      }

      if (do_export && e0 < s.p_export) {
        float gs = 0.f;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const int r = m / G, h = g * G + m % G;
            const float l = acc[m] * a.scale;
            if (e < s.p_export && a.logits) {
              if (a.export_all) {
                a.logits[((size_t)(b * a.nrows + r) * Hq + h) * a.max_prefix + e] = l;
              } else {
                if (r == 0) a.logits[((size_t)(b * 2 + 0) * Hq + h) * a.max_prefix + e] = l;
                if (r == a.gamma) a.logits[((size_t)(b * 2 + 1) * Hq + h) * a.max_prefix + e] = l;
              }
            }
            gs += (a.export_all ? 1.f : (float)((r == 0) + (r == a.gamma))) * acc[m];
          }
        }
        if (a.group && e < s.p_export) a.group[(size_t)(b * Hkv + g) * a.max_prefix + e] = gs * a.scale;
      }

      // Softmax with the wave reductions on DPP / lane swaps (no LDS round
      // trips); the running max and rescale factor are wave-uniform.  The
      // scaled logit is rounded once (no multiply-add contraction into the
      // exponent's argument), so the entry that sets the maximum gets p = 1.
      float alpha[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int vis = s.vis0 + m / G;
        const bool ok = (e < e_end) && (e < vis);
        const float x = ok ? __fmul_rn(acc[m], a.scale_log2) : kNegInf;
        const float m_new = first_lane(fmaxf(m_run[m], wave_max_dpp(x)));
        alpha[m] = first_lane(exp2_fast(m_run[m] - m_new));
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
      // PV over all 64 entries (masked ones have p = 0 and a real row);
      // probabilities broadcast from LDS, 4 entries per read
#pragma unroll
      for (int j4 = 0; j4 < kWave; j4 += 4) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&sm.loop.p[wave][m][j4]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < DV; ++k) o[m][k] = fmaf(p4[i], vv[j4 + i][k], o[m][k]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    __syncthreads();  // the merge area aliases the loop buffers
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float lsum = sum_across_groups(sum_within_group(l_run[m]));
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
