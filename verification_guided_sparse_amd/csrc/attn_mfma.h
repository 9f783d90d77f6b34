// attn_mfma.h -- bf16 attention over paged key lists on the CDNA4 matrix cores
// (v_mfma_f32_16x16x32_bf16), used for both verification attention (all
// cache positions, causal among the new rows, logit export) and sparse draft
// attention (selected slots + causal tail).
//
// The 32-entry tiles of all (sequence b, KV head g) key lists are shared
// evenly among the workgroups (attn_common.h); a workgroup = 4 waves walks its
// share piece by piece, a piece being the part of the share inside one list.
// For a piece the query rows of KV head g (M = nrows * G, padded to NT tiles of
// 16) stay in registers; each wave takes the piece's tiles t = wave, wave + 4,
// ...:
//
//   S^T[tok][row] = K[tok][:] . Q[row][:]     A = K rows straight from HBM,
//                                             B = Q^T held in registers
//   online softmax over tok, per row          (log2 domain, fp32)
//   O^T[d][row] += V^T[d][tok] P^T[tok][row]  A = V^T built in registers from
//                                             full-row V loads, B = P^T (bf16)
//
// Lane l = 16*q4 + i16.  MFMA 16x16x32 operands: lane holds A[i16][8*q4 .. +7]
// and B[8*q4 .. +7][i16]; the result C[4*q4 + c][i16], c = 0..3.
//  * K: rows are read whole (CH = D/8 lanes x 16 bytes per row, 64/CH rows
//    per instruction) and parked in a per-wave LDS tile whose rows are padded
//    to D*2 + 16 bytes, so that both this write and the operand read are free
//    of bank conflicts.  The operand read gives lane (q4, i16) token
//    tt*16 + i16, d-chunk 4*ks + q4: the contraction over d may visit d in any
//    order as long as Q uses the same one.  (Reading K straight into operand
//    layout makes 64-byte fragments per token and measurably less HBM
//    bandwidth than whole-row reads.)
//  * V: lane loads d-chunk i16 of the 8 tokens tok(q4, v); 16 lanes cover one
//    full 256-byte (D = 128) or 128-byte (D = 64) row per instruction.  Their
//    8 x 8 (or 8 x 4) bf16 are repacked with byte permutes so that MFMA tile
//    `at` holds d = DPL*i16 + at for the 8 tokens.
//  * tok(q4, v) = v < 4 ? 4*q4 + v : 16 + 4*q4 + (v - 4) is exactly the token
//    set lane (q4, i16) holds in the S^T result, so P^T needs no lane movement.
//  * Exports (verify): a tile's group sums, and at D = 128 its raw logits, go
//    to an LDS staging area and leave as contiguous nontemporal runs at the
//    end of each chunk of the piece (see the kernel).
#pragma once

#include "attn_common.h"

namespace vg {

template <int D>
struct VRow;  // one lane's slice of one V row
template <>
struct VRow<128> {
  u32x4 w;  // d = 8*i16 .. 8*i16 + 7
};
template <>
struct VRow<64> {
  u32x2 w;  // d = 4*i16 .. 4*i16 + 3
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return (x & 0xffffu) | (y << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return (x >> 16) | (y & 0xffff0000u);
}

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// One 32-entry tile of K and V for this lane (see the layout notes above).
template <int D>
struct KVTile {
  u32x4 kraw[D / 16];  // whole-row K loads: instruction i holds rows i*(64/CH) + lane/CH
  VRow<D> vr[8];
};

// Per-wave LDS staging of one K tile: 32 rows padded to D*2 + 16 bytes.
// A16: the rows are declared 16-byte aligned, so the compiler moves the tile
// through LDS with 128-bit accesses instead of pairs of 32-bit ones.  Measured
// on the same box: that makes a 128K draft step about 1 % faster and the
// verify call 1-3 % slower, so only the sparse kernels declare it.
template <int D, bool A16>
struct KStage {
  static constexpr int kRowBytes = D * 2 + 16;
  alignas(A16 ? 16 : 1) char rows[32 * kRowBytes];
};

// Slots of a chunk of a piece's entries, staged in LDS once per workgroup so
// that the tile loop issues its K/V loads without a dependent page-table load.
//   verify: page ids of the chunk's pages (entry e -> slot_sm[e/16 - page0] * 16 + e % 16)
//   sparse: the chunk's part of the explicit slot list (entries below cnt)
constexpr int kSlotSm = 1024;

__device__ __forceinline__ void stage_slots(int *slot_sm, const AttnArgs &a, int b, const SeqList &s,
                                            int e_begin, int e_end) {
  if (!a.sparse) {
    const int p0 = e_begin >> 4, n = ((e_end - 1) >> 4) - p0 + 1;
    for (int i = threadIdx.x; i < n; i += kThreads)
      slot_sm[i] = a.page_table[(size_t)b * a.max_pages + p0 + i];
  } else {
    const int n = min(e_end, s.cnt) - e_begin;
    for (int i = threadIdx.x; i < n; i += kThreads)
      slot_sm[i] = a.sel_slot[(size_t)b * a.max_k + e_begin + i];
  }
}

// Entries staged per chunk of a piece: verify stages page ids (1 per 16
// entries), sparse stages slots (1 per entry).  Each chunk boundary drains
// the tile pipeline (about 3 us), so the D = 128 verify kernels without the
// raw export have a long-chunk form (kSlotSm pages, twice the group-sum
// staging) for calls whose workgroup shares exceed one chunk; it is not the
// default because the larger LDS allocation costs a short-share call (one
// chunk per workgroup) about half a microsecond.
constexpr int kVerifyChunk = kSlotSm / 2 * kPageSize;
constexpr int kVerifyChunkLong = kSlotSm * kPageSize;
constexpr int kSparseChunk = kSlotSm;

// Raw-logit rows staged per chunk (D = 128 kernels): at most kRawStage
// logits (rows x positions, 64 KB) plus 4 floats of padding per row (rows 16
// bytes apart in bank order, so that a tile's 16 rows are written without
// LDS bank conflicts).  Staging is used when the chunk it allows holds at
// least kRawStageMin entries (two rows per query head); with more rows
// (every row exported) the chunks would be so short that restarting the tile
// pipeline at each one costs more than it saves, and the rows are stored per
// tile, as in the D = 64 kernels (two workgroups per CU leave no room).
constexpr int kRawStage = 16384;
constexpr int kRawStagePad = 4;
constexpr int kRawStageMin = 1024;

// Chunk length of a verify piece with nx staged raw-logit rows: the largest
// multiple of the 32-entry tile whose nx rows fit the staging area, at most
// kVerifyChunk.
__host__ __device__ constexpr int raw_chunk(int nx) {
  return ((kRawStage / nx) & ~31) < kVerifyChunk ? ((kRawStage / nx) & ~31) : kVerifyChunk;
}

// LDS of the tile loop: the waves' K staging areas and NS floats of export
// staging (the chunk's group sums, then its raw-logit rows).
template <int D, bool A16, int NS>
struct LoopSmem {
  KStage<D, A16> kst[kWaves];
  float st[NS];
  __device__ float *staging() { return st; }
};
template <int D, bool A16>
struct LoopSmem<D, A16, 0> {
  KStage<D, A16> kst[kWaves];
  __device__ float *staging() { return nullptr; }  // (never dereferenced)
};

__device__ __forceinline__ int staged_slot(const int *slot_sm, const AttnArgs &a, int b,
                                           const SeqList &s, int e_begin, int e) {
  if (!a.sparse) return slot_sm[(e >> 4) - (e_begin >> 4)] * kPageSize + (e & (kPageSize - 1));
  if (e < s.cnt) return slot_sm[e - e_begin];
  return entry_slot(a, b, s, e);  // causal tail: a few positions through the page table
}

template <int D>
__device__ __forceinline__ void load_tile(KVTile<D> &T, const AttnArgs &a, int b, const SeqList &s,
                                          int e0, int g, int lane, const int *slot_sm, int e_begin,
                                          int e_end, bool pref = false, int pf_slot = 0, int jt = 0) {
  constexpr int DPL = D / 16;
  const int q4 = lane >> 4, i16 = lane & 15;
  // A slot is a row index of the cache (non-negative, below 2^31) and a row
  // is at most a few KB, so a row's byte offset is one 32 x 32 -> 64-bit
  // multiply-add (a 64-bit product would take three quarter-rate multiplies
  // per load address).
  const uint32_t slot_bytes = (uint32_t)a.num_kv_heads * D * 2;
  const size_t head_off = (size_t)g * D * 2;
  // slot of entry e0 + (lane & 31); each lane then picks the slots it loads.
  // Entries past the chunk's end (masked later) reuse its last entry, whose
  // slot is staged.
  const int my_e = min(e0 + (lane & 31), e_end - 1);
  // prefetched split: lane l of this wave holds the slot of entry l & 31 of
  // its tile (l >> 5)
  const int rs = __shfl(pf_slot, ((my_e - e0) + 32 * jt) & 63);  // (every lane takes part)
  const int my_slot = pref ? (my_e < s.cnt ? rs : entry_slot(a, b, s, my_e)) : staged_slot(slot_sm, a, b, s, e_begin, my_e);
  const char *kc = static_cast<const char *>(a.k_cache);
  const char *vc = static_cast<const char *>(a.v_cache);
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CH;    // rows per instruction
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int row = i * RPI + lane / CH;
    const int ks_slot = __shfl(my_slot, row);
    const char *krow = kc + (uint64_t)(uint32_t)ks_slot * slot_bytes + head_off + (lane % CH) * 16;
    T.kraw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(krow));
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int vs = __shfl(my_slot, v < 4 ? 4 * q4 + v : 12 + 4 * q4 + v);
    const char *vrow = vc + (uint64_t)(uint32_t)vs * slot_bytes + head_off + i16 * (DPL * 2);
    if constexpr (D == 128)
      T.vr[v].w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vrow));
    else
      T.vr[v].w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(vrow));
  }
}

template <int D, int NT>
struct WaveState {
  u32x4 qf[NT][D / 32];  // Q^T fragments (B operand of S^T = K Q^T)
  f32x4 o[NT][D / 16];   // O^T accumulators
  float m_run[NT], l_run[NT];
  // per-lane constants of this lane's rows (row = rt*16 + i16)
  int vis_off[NT];       // the row sees entries i < s.vis0 + vis_off
  int head[NT];          // its query head, -1 for padding rows
  float gw[NT];          // weight of the row in the group export: #{r in {0, gamma}} (every row: 1)
  int xrow[NT];          // export slots: bit x -> slot xbase + x of the raw export
  int xbase[NT];         // 0, or the row r when every row is exported
};

// GST: the group sums go to the chunk's LDS staging area `gst` (entry e at
// gst[e - gc0]) instead of straight to memory; RAW kernels stage their
// raw-logit rows likewise in `xst` (row xr = slot * G + head in group, xs
// floats apart).
template <int D, int NT, bool RAW, bool A16, bool GST, bool XST>
__device__ __forceinline__ void compute_tile(WaveState<D, NT> &W, const KVTile<D> &T,
                                             KStage<D, A16> &ks_sm, const AttnArgs &a, int b, int g,
                                             const SeqList &s, int e0, int e_end, int lane,
                                             bool do_export, bool vec_export, float *gst, int gc0,
                                             float *xst, int xs) {
  constexpr int KS = D / 32, DPL = D / 16;
  constexpr int CH = D / 8, RPI = 64 / CH, RB = KStage<D, A16>::kRowBytes;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int Hkv = a.num_kv_heads;

  // K rows -> LDS -> operand layout (this wave's staging area only)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int row = i * RPI + lane / CH;
    *reinterpret_cast<u32x4 *>(ks_sm.rows + row * RB + (lane % CH) * 16) = T.kraw[i];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  u32x4 kf[2][KS];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[tt][ks] = *reinterpret_cast<const u32x4 *>(ks_sm.rows + (tt * 16 + i16) * RB + (4 * ks + q4) * 16);

  // S^T = K Q^T
  f32x4 st[2][NT];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[tt][ks]), as_bf16x8(W.qf[rt][ks]),
                                                      acc, 0, 0, 0);
      st[tt][rt] = acc;
    }

  // Logit export (verify): rows 0 and gamma (or every row), entries below the
  // prefix length.
  if (do_export && e0 < s.p_export) {
    if (RAW && a.logits) {  // staged (xst set: the chunk's rows are written at its end) or stored here
      const int Hq = a.num_q_heads;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        if (W.xrow[rt]) {
          const int h = W.head[rt];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (W.xrow[rt] & (1 << x)) {
              const int slot = W.xbase[rt] + x;
              if (XST && xst) {
                float *xrow = xst + (slot * a.group_size + (h - g * a.group_size)) * xs;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                  const int e = e0 + tt * 16 + 4 * q4;
                  *reinterpret_cast<f32x4 *>(xrow + (e - gc0)) = st[tt][rt] * a.scale;
                }
              } else {
                const int n_slots = a.export_all ? a.nrows : 2;
                float *dst = a.logits + ((size_t)(b * n_slots + slot) * Hq + h) * a.max_prefix;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                  const int e = e0 + tt * 16 + 4 * q4;
                  const f32x4 lv = st[tt][rt] * a.scale;
                  if (vec_export && e + 3 < s.p_export) {
                    *reinterpret_cast<f32x4 *>(dst + e) = lv;
                  } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                      if (e + c < s.p_export) dst[e + c] = lv[c];
                  }
                }
              }
            }
          }
        }
      }
    }
    if (a.group) {
      float *dst = a.group + (size_t)(b * Hkv + g) * a.max_prefix;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 gs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) gs += W.gw[rt] * st[tt][rt];
#pragma unroll
        for (int c = 0; c < 4; ++c) gs[c] = sum_within_group(gs[c]) * a.scale;
        if (i16 == 0) {
          const int e = e0 + tt * 16 + 4 * q4;
          if (GST) {
            *reinterpret_cast<f32x4 *>(gst + (e - gc0)) = gs;
          } else if (vec_export && e + 3 < s.p_export) {
            *reinterpret_cast<f32x4 *>(dst + e) = gs;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (e + c < s.p_export) dst[e + c] = gs[c];
          }
        }
      }
    }
  }

  // Online softmax (base 2) and P^T fragments.  The scaled logits are rounded
  // once (no multiply-add contraction into the exponent's argument), so the
  // entry that sets the running maximum gets p = 1 exactly.  Masking is only needed on
  // tiles that reach past the chunk's end or into the causal part of the key
  // list; O is rescaled only if some row's running maximum grew (otherwise
  // every alpha is exactly 1).
  const bool full = (e0 + 32 <= e_end) && (e0 + 32 <= s.vis0);
  bf16x8 pb[NT];
  float alpha[NT];
  bool grew = false;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    float x[2][4];
    float mx = kMInit;
    if (full) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[tt][c] = __fmul_rn(st[tt][rt][c], a.scale_log2);
          mx = fmaxf(mx, x[tt][c]);
        }
    } else {
      const int vis = s.vis0 + W.vis_off[rt];  // entries i < vis are visible to this row
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = e0 + tt * 16 + 4 * q4 + c;
          const bool ok = (e < e_end) && (e < vis);
          x[tt][c] = ok ? __fmul_rn(st[tt][rt][c], a.scale_log2) : kNegInf;
          mx = fmaxf(mx, x[tt][c]);
        }
    }
    mx = max_across_groups(mx);
    const float m_new = fmaxf(W.m_run[rt], mx);
    grew |= m_new > W.m_run[rt];
    alpha[rt] = exp2_fast(W.m_run[rt] - m_new);
    W.m_run[rt] = m_new;
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[tt][c] = exp2_fast(x[tt][c] - m_new);
        psum += p[tt][c];
      }
    W.l_run[rt] = W.l_run[rt] * alpha[rt] + psum;
    u32x4 pk;
    pk[0] = f32x2_to_bf16x2(p[0][0], p[0][1]);
    pk[1] = f32x2_to_bf16x2(p[0][2], p[0][3]);
    pk[2] = f32x2_to_bf16x2(p[1][0], p[1][1]);
    pk[3] = f32x2_to_bf16x2(p[1][2], p[1][3]);
    pb[rt] = as_bf16x8(pk);
  }
  if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int at = 0; at < DPL; ++at) W.o[rt][at] *= alpha[rt];
  }

  // O^T += V^T P^T
#pragma unroll
  for (int at = 0; at < DPL; ++at) {
    u32x4 va;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x0 = T.vr[2 * w].w[at >> 1], x1 = T.vr[2 * w + 1].w[at >> 1];
      va[w] = (at & 1) ? pack_hi(x0, x1) : pack_lo(x0, x1);
    }
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
      W.o[rt][at] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb[rt], W.o[rt][at], 0, 0, 0);
  }
}

// RAW: the raw-logit export is compiled in (verify calls that export raw
// logits); without it the kernel exports group sums only, or nothing.
// LONGC: verify chunks of kVerifyChunkLong entries (D = 128 without RAW).
template <int D, int NT, int PF, bool SPARSE, bool RAW = false, bool LONGC = false>
__global__ __launch_bounds__(kThreads, attn_occupancy(D, NT, PF, SPARSE))
void attn_mfma_kernel(AttnArgs a_in) {
  AttnArgs a = a_in;
  a.sparse = SPARSE ? 1 : 0;
  constexpr int KS = D / 32;   // k-steps of the QK^T contraction
  constexpr int DPL = D / 16;  // d values per lane per V row, = number of PV tiles
  constexpr int ROWS = NT * 16;
  // Exports staged per chunk (verify kernels): a tile's group sums and (at
  // D = 128) raw logits go to LDS, and each of the chunk's rows is written at
  // the chunk's end as one contiguous run with nontemporal stores.  Written
  // straight from each tile (128 bytes of a row at a time, spread over all
  // workgroups' rows), the lines reach HBM one by one in the middle of the
  // K/V read stream and cost far more than their bytes.  The D = 64 kernels
  // run two workgroups per CU and leave no LDS for raw rows, which they
  // store per tile.
  constexpr bool GST = !SPARSE;
  constexpr bool XST = RAW && !SPARSE && D == 128;
  static_assert(!LONGC || (D == 128 && !RAW && !SPARSE), "long chunks: D = 128 verify kernels without RAW");
  constexpr int VCH = LONGC ? kVerifyChunkLong : kVerifyChunk;  // longest verify chunk
  constexpr int NS = (GST ? VCH : 0) + (XST ? kRawStage + kRawStagePad * kMaxRows : 0);
  __shared__ union {
    LoopSmem<D, SPARSE, NS> t;  // during the tile loop
    MergeSmem<ROWS, D> m;       // after it
  } lds;
  MergeSmem<ROWS, D> &sm = lds.m;
  __shared__ int slot_sm[kSlotSm];
  __shared__ int pre[kMaxBatch + 1];
  __shared__ int lens[kMaxBatch];
  __shared__ int sm4[4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int G = a.group_size, M = a.rows, Hq = a.num_q_heads;
  const bool do_export = !a.sparse && (a.logits != nullptr || a.group != nullptr);
  const bool vec_export = (a.max_prefix & 3) == 0;
  // raw-logit rows of this KV head (two per query head, or every row), and
  // whether they are staged (then with a shorter chunk and this LDS stride)
  const int nx = (RAW && a.logits) ? (a.export_all ? a.nrows : 2) * G : 0;
  const bool xstage = XST && nx > 0 && raw_chunk(nx) >= kRawStageMin;
  const int chunk = a.sparse ? kSparseChunk : xstage ? raw_chunk(nx) : VCH;
  const int xs = chunk + kRawStagePad;
  float *const gst = lds.t.staging();
  float *const xst = lds.t.staging() + (GST ? VCH : 0);
  // Fixed sparse splits (at most kThreads entries, one chunk): this
  // workgroup's part of the explicit slot list is loaded now, together with
  // the list length rather than after it, straight into the registers of the
  // waves that load those entries' K/V rows (no LDS staging, no barrier).
  // Entries past the selection count are loaded (they are inside the
  // [B][max_k] list) but never used.
  const bool pref = a.sparse && a.split_tokens > 0 && a.split_tokens <= kThreads;
  int pf_slot = 0;
  if (pref) {  // lane l of wave v: entry 32 (v + 4 (l >> 5)) + (l & 31) of the split (its tile l >> 5)
    const int seg = blockIdx.x / a.splits;
    const int le = 32 * (((int)threadIdx.x >> 6) + kWaves * (((int)threadIdx.x >> 5) & 1)) + ((int)threadIdx.x & 31);
    const int e = (blockIdx.x % a.splits) * a.split_tokens + le;
    if (le < a.split_tokens && e < a.max_k)
      pf_slot = a.sel_slot[(size_t)(seg / a.num_kv_heads) * a.max_k + e];
  }

  // Query fragments of (sequence b, KV head g): lane (q4, i16) holds row
  // rt * 16 + i16, d-chunks 4 * ks + q4.
  auto load_q = [&](int b, int g, u32x4 (&qf)[NT][KS]) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const int row = rt * 16 + i16;
      if (row < M) {
        const int r = row / G, h = g * G + row % G;
        const uint16_t *qrow =
            static_cast<const uint16_t *>(a.q) + ((size_t)(b * a.nrows + r) * Hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = *reinterpret_cast<const u32x4 *>(qrow + (4 * ks + q4) * 8);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // With fixed sparse splits the queries too are loaded before the list length.
  u32x4 q_pre[NT][KS];
  if (pref) {
    const int seg = blockIdx.x / a.splits;
    load_q(seg / a.num_kv_heads, seg % a.num_kv_heads, q_pre);
  }

  for_each_piece(a, pre, lens, sm4, [&](int b, int g, int part, int e_begin, int e_end) {
    const SeqList s = seq_list(a, b);
    WaveState<D, NT> W;
    if (pref) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) W.qf[rt][ks] = q_pre[rt][ks];
    } else {
      load_q(b, g, W.qf);
    }
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const int row = rt * 16 + i16;
      W.m_run[rt] = kMInit;
      W.l_run[rt] = 0.f;
      const int r = row / G;
      W.vis_off[rt] = r;
      W.head[rt] = row < M ? g * G + row % G : -1;
      if (a.export_all) {
        W.gw[rt] = row < M ? 1.f : 0.f;
        W.xrow[rt] = row < M ? 1 : 0;
        W.xbase[rt] = r;
      } else {
        W.gw[rt] = row < M ? (float)((r == 0) + (r == a.gamma)) : 0.f;
        W.xrow[rt] = row < M ? ((r == 0) | ((r == a.gamma) << 1)) : 0;
        W.xbase[rt] = 0;
      }
#pragma unroll
      for (int at = 0; at < DPL; ++at) W.o[rt][at] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int c0 = e_begin; c0 < e_end; c0 += chunk) {
      const int c1 = min(e_end, c0 + chunk);
      if (!pref) {  // (a prefetched split is one chunk whose slots are in registers)
        __syncthreads();  // earlier users of slot_sm / the K staging area are done
        stage_slots(slot_sm, a, b, s, c0, c1);
        __syncthreads();
      }
      // This wave's tiles: j = 0 .. nw-1 cover entries c0 + 32 * (wave + 4 j).
      const int ntiles = (c1 - c0 + 31) / 32;
      const int nw = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
      auto e_of = [&](int j) { return c0 + 32 * (wave + kWaves * j); };
      // PF tiles in flight per wave: tile j + PF loads while tile j computes.
      // In the steady state every load is issued unconditionally, so the wait
      // before a tile covers exactly that tile's (oldest) loads.
      KVTile<D> T[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u)
        if (u < nw) load_tile<D>(T[u], a, b, s, e_of(u), g, lane, slot_sm, c0, c1, pref, pf_slot, u);
      int j = 0;
      for (; j + 2 * PF <= nw; j += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          compute_tile<D, NT, RAW, SPARSE, GST, XST>(W, T[u], lds.t.kst[wave], a, b, g, s, e_of(j + u), c1, lane, do_export, vec_export, gst, c0, xstage ? xst : nullptr, xs);
          load_tile<D>(T[u], a, b, s, e_of(j + u + PF), g, lane, slot_sm, c0, c1, pref, pf_slot, j + u + PF);
        }
      }
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (j + u < nw) {
          compute_tile<D, NT, RAW, SPARSE, GST, XST>(W, T[u], lds.t.kst[wave], a, b, g, s, e_of(j + u), c1, lane, do_export, vec_export, gst, c0, xstage ? xst : nullptr, xs);
          if (j + u + PF < nw) load_tile<D>(T[u], a, b, s, e_of(j + u + PF), g, lane, slot_sm, c0, c1, pref, pf_slot, j + u + PF);
        }
      }
#pragma unroll
      for (int u = 0; u < PF; ++u)
        if (j + PF + u < nw)
          compute_tile<D, NT, RAW, SPARSE, GST, XST>(W, T[u], lds.t.kst[wave], a, b, g, s, e_of(j + PF + u), c1, lane, do_export, vec_export, gst, c0, xstage ? xst : nullptr, xs);
      // the chunk's staged exports, entries below the prefix length
      if ((GST && a.group || xstage) && c0 < s.p_export) {
        __syncthreads();
        const int n = min(c1, s.p_export) - c0, n4 = (n + 3) >> 2;
        auto put = [&](float *dst, const float *src, int i) {  // entries i .. i+3 of the run
          const f32x4 v = *reinterpret_cast<const f32x4 *>(src + i);
          if (vec_export && i + 3 < n) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dst + i));
          } else {
            for (int c = 0; c < 4; ++c)
              if (i + c < n) dst[i + c] = v[c];
          }
        };
        if (GST && a.group) {
          float *dst = a.group + (size_t)(b * a.num_kv_heads + g) * a.max_prefix + c0;
          for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * kThreads) put(dst, gst, i);
        }
        if (xstage) {  // row xr = slot * G + head in group
          const int n_slots = a.export_all ? a.nrows : 2;
          for (int k = threadIdx.x; k < nx * n4; k += kThreads) {
            const int xr = k / n4, i = 4 * (k - xr * n4);
            const int slot = xr / G, h = g * G + (xr - slot * G);
            float *dst = a.logits + ((size_t)(b * n_slots + slot) * Hq + h) * a.max_prefix + c0;
            put(dst, xst + xr * xs, i);
          }
        }
      }
    }

    __syncthreads();  // the K staging area becomes the merge area
    // Merge the 4 waves' states into this piece's partial.
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const float lsum = sum_across_groups(W.l_run[rt]);
      if (q4 == 0) {
        sm.m[wave][rt * 16 + i16] = W.m_run[rt];
        sm.l[wave][rt * 16 + i16] = lsum;
      }
    }
    __syncthreads();
    const size_t pidx = (size_t)part * M;
    const RowStat st = merge_stats<ROWS, D>(sm);
    // O^T tile `at`, register c holds row (rt*16 + i16), d = DPL*(4*q4 + c) + at.
    // Only the M real rows are written (the draft has 4 of a tile's 16).
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      float *orow = &sm.o[wave][rt * 16 + i16][0];
      if (rt * 16 + i16 >= M) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = DPL * (4 * q4 + c);
#pragma unroll
        for (int at = 0; at < DPL; at += 4)
          *reinterpret_cast<f32x4 *>(orow + d0 + at) =
              f32x4{W.o[rt][at][c], W.o[rt][at + 1][c], W.o[rt][at + 2][c], W.o[rt][at + 3][c]};
      }
    }
    __syncthreads();
    merge_o<ROWS, D>(sm, a.part_o + pidx * D, M);
    store_stats(a.part_ml + pidx * 2, M, st);
  });
}

}  // namespace vg
