// select.h -- score aggregation and exact top-k selection.
//
// Scores map to order-preserving 32-bit keys (larger score <-> larger key;
// -0.0 is folded onto +0.0).  The k-th largest key K* is found by a radix
// select over key bits [20,32) / [10,20) / [0,10):
//
//   pass 1  (one workgroup per 2048 positions): LDS histogram of bits
//           [20,32), merged into a per-sequence global histogram with
//           atomics.  Optionally fused with the aggregation that produces the
//           scores.
//   pass 2  (one workgroup per 2048 positions): every workgroup reads the
//           global histogram and finds the bin b1 that holds K*, then stages,
//           in ascending position order, each entry whose bin is >= b1 (the
//           sure picks and the candidates of bin b1).  The last workgroup of
//           the sequence clears the histogram, resolves bits [10,20) and
//           [0,10) on the candidates, and walks the staged entries in
//           position order: it keeps keys > K* and the first (k - #keys > K*)
//           keys equal to K*, writing positions ascending and their
//           page-size-1 slots.
//
// The histogram and the completion counters are left at zero after each call.
#pragma once

#include "vg_device.h"

namespace vg {

constexpr int kSelThreads = 256;
constexpr int kChunk = 2048;                   // positions per pass workgroup
constexpr int kPerThread = kChunk / kSelThreads;  // 8 consecutive positions per thread
constexpr int kBins1 = 4096;                   // key bits [20, 32)
constexpr int kBins23 = 1024;                  // key bits [10, 20), then [0, 10)
constexpr int kMaxChunks = 1024;               // max_prefix <= 2^21

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workspace of one selection (per sequence b):
//   hist1 [B][kBins1] u32   zero at rest
//   done  [B] u32           zero at rest
//   ccount[B][kMaxChunks] i32
//   stage [B][max_prefix] u32x2 (key, position)
struct SelWs {
  uint32_t *hist1;
  uint32_t *done;
  int32_t *ccount;
  u32x2 *stage;
};

struct SelArgs {
  int32_t batch, max_prefix, max_k;
  const int32_t *prefix_len;
  const int32_t *k;
  const float *scores;        // pass 1 (unfused) and pass 2 read these
  float *scores_out;          // fused aggregation writes them
  const float *src;           // aggregation source [B][rows][heads][max_prefix]
  int32_t src_rows, src_heads;
  const int32_t *page_table;
  int32_t page_size, max_pages;
  int32_t *sel_pos, *sel_slot, *sel_count;
  SelWs ws;
};

// Exclusive prefix sum over a 256-thread block; `total` receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int *sm4, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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

// Given a histogram in LDS (nbins, higher bin = larger key) and a rank k >= 1,
// find the bin holding the k-th largest key.  Returns the bin and, in `above`,
// the number of keys in higher bins.  Block-wide; every thread gets the result.
__device__ __forceinline__ int find_bin(const uint32_t *h, int nbins, int k, int *sm4, int *sm_res,
                                        int &above) {
  const int per = nbins / kSelThreads;  // bins per thread (4 or 16)
  const int t = threadIdx.x;
  // thread t owns bins [nbins - per*(t+1), nbins - per*t), scanned from the top
  const int top = nbins - per * t;
  int local = 0;
  for (int i = 1; i <= per; ++i) local += (int)h[top - i];
  int total;
  const int pre = block_exclusive_scan(local, sm4, total);
  if (t == 0) {
    sm_res[0] = 0;
    sm_res[1] = 0;
  }
  __syncthreads();
  if (pre < k && k <= pre + local) {
    int run = pre;
    for (int i = 1; i <= per; ++i) {
      const int c = (int)h[top - i];
      if (k <= run + c) {
        sm_res[0] = top - i;
        sm_res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  above = sm_res[1];
  const int bin = sm_res[0];
  __syncthreads();
  return bin;
}

// Pass 1.  grid (nchunks, B).  AGG: compute scores from src and write them.
// HIST: add the chunk's bits [20,32) histogram to the global one.
template <bool AGG, bool HIST>
__global__ __launch_bounds__(kSelThreads) void select_pass1_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins1];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = a.prefix_len[b];
  const int nch = (P + kChunk - 1) / kChunk;
  if (w >= nch) return;
  if (HIST) {
    for (int i = t; i < kBins1; i += kSelThreads) lh[i] = 0u;
    __syncthreads();
  }
  const int j0 = w * kChunk + t * kPerThread;
  float sc[kPerThread];
  if (AGG) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) sc[i] = 0.f;
    const bool vec = ((a.max_prefix & 3) == 0) && (j0 + kPerThread <= P);
    for (int r = 0; r < a.src_rows; ++r)
      for (int h = 0; h < a.src_heads; ++h) {
        const float *row = a.src + ((size_t)(b * a.src_rows + r) * a.src_heads + h) * a.max_prefix;
        if (vec) {
          const f32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + j0));
          const f32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + j0 + 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[i] += v0[i];
            sc[4 + i] += v1[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < kPerThread; ++i)
            if (j0 + i < P) sc[i] += row[j0 + i];
        }
      }
    float *dst = a.scores_out + (size_t)b * a.max_prefix;
    if (vec) {
      *reinterpret_cast<f32x4 *>(dst + j0) = f32x4{sc[0], sc[1], sc[2], sc[3]};
      *reinterpret_cast<f32x4 *>(dst + j0 + 4) = f32x4{sc[4], sc[5], sc[6], sc[7]};
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i)
        if (j0 + i < P) dst[j0 + i] = sc[i];
    }
  } else {
    const float *srow = a.scores + (size_t)b * a.max_prefix;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) sc[i] = (j0 + i < P) ? srow[j0 + i] : 0.f;
  }
  if (!HIST) return;

#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (j0 + i < P) atomicAdd(&lh[score_key(sc[i]) >> 20], 1u);
  __syncthreads();
  uint32_t *gh = a.ws.hist1 + (size_t)b * kBins1;
  for (int i = t; i < kBins1; i += kSelThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Pass 2.  grid (nchunks, B).
__global__ __launch_bounds__(kSelThreads) void select_pass2_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins1];
  __shared__ int csum[kMaxChunks + 1];
  __shared__ int sm4[4];
  __shared__ int sm_res[2];
  __shared__ int sm_last;
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = a.prefix_len[b];
  const int k_eff = min(a.k[b], P);
  if (P <= 0) {
    if (w == 0 && t == 0) a.sel_count[b] = 0;
    return;
  }
  const int nch = (P + kChunk - 1) / kChunk;
  if (w >= nch) return;
  uint32_t *gh = a.ws.hist1 + (size_t)b * kBins1;
  u32x2 *stage = a.ws.stage + (size_t)b * a.max_prefix;

  // The bin of K* from the complete pass-1 histogram.
  uint32_t b1 = 0xffffffffu;  // k_eff == 0: stage nothing
  int above1 = 0;
  if (k_eff > 0) {
    for (int i = t; i < kBins1; i += kSelThreads) lh[i] = gh[i];
    __syncthreads();
    b1 = (uint32_t)find_bin(lh, kBins1, k_eff, sm4, sm_res, above1);
  }

  // Stage entries with bin >= b1 in ascending position order.
  const int j0 = w * kChunk + t * kPerThread;
  const float *srow = a.scores + (size_t)b * a.max_prefix;
  uint32_t key[kPerThread];
  int nflag = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    key[i] = (j0 + i < P) ? score_key(srow[j0 + i]) : 0u;
    nflag += (j0 + i < P) && ((key[i] >> 20) >= b1);
  }
  int total;
  int off = block_exclusive_scan(nflag, sm4, total);
  u32x2 *cst = stage + (size_t)w * kChunk;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if ((j0 + i < P) && ((key[i] >> 20) >= b1)) cst[off++] = u32x2{key[i], (uint32_t)(j0 + i)};
  if (t == 0) a.ws.ccount[(size_t)b * kMaxChunks + w] = total;

  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t ticket = atomicAdd(&a.ws.done[b], 1u);
    sm_last = (ticket == (uint32_t)(nch - 1));
  }
  __syncthreads();
  if (!sm_last) return;
  __threadfence();
  // every workgroup has read the histogram: clear it for the next call
  for (int i = t; i < kBins1; i += kSelThreads) gh[i] = 0u;
  if (k_eff <= 0) {
    if (t == 0) {
      a.sel_count[b] = 0;
      atomicExch(&a.ws.done[b], 0u);
    }
    return;
  }

  // ---- last block of sequence b: resolve K* and write the selection ----
  // chunk prefix sums of the staged counts
  {
    int local = 0;
    const int per = (nch + kSelThreads - 1) / kSelThreads;
    for (int i = 0; i < per; ++i) {
      const int c = t * per + i;
      local += (c < nch) ? __hip_atomic_load(&a.ws.ccount[(size_t)b * kMaxChunks + c],
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0;
    }
    int tot;
    int run = block_exclusive_scan(local, sm4, tot);
    for (int i = 0; i < per; ++i) {
      const int c = t * per + i;
      if (c < nch) {
        csum[c] = run;
        run += __hip_atomic_load(&a.ws.ccount[(size_t)b * kMaxChunks + c], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (t == 0) csum[nch] = tot;
    __syncthreads();
  }
  const int n_st = csum[nch];
  // staged entry number gi -> (chunk, index): largest c with csum[c] <= gi
  auto staged = [&](int gi) -> u32x2 {
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (csum[mid] <= gi) lo = mid; else hi = mid - 1;
    }
    return stage[(size_t)lo * kChunk + (gi - csum[lo])];
  };

  // bits [10, 20) among candidates (bin == b1)
  int k1 = k_eff - above1;  // >= 1: rank of K* inside bin b1
  for (int i = t; i < kBins23; i += kSelThreads) lh[i] = 0u;
  __syncthreads();
  for (int gi = t; gi < n_st; gi += kSelThreads) {
    const u32x2 e = staged(gi);
    if ((e[0] >> 20) == b1) atomicAdd(&lh[(e[0] >> 10) & 1023u], 1u);
  }
  __syncthreads();
  int above2;
  const uint32_t b2 = (uint32_t)find_bin(lh, kBins23, k1, sm4, sm_res, above2);
  const int k2 = k1 - above2;
  const uint32_t pre21 = (b1 << 10) | b2;
  for (int i = t; i < kBins23; i += kSelThreads) lh[i] = 0u;
  __syncthreads();
  for (int gi = t; gi < n_st; gi += kSelThreads) {
    const u32x2 e = staged(gi);
    if ((e[0] >> 10) == pre21) atomicAdd(&lh[e[0] & 1023u], 1u);
  }
  __syncthreads();
  int above3;
  const uint32_t b3 = (uint32_t)find_bin(lh, kBins23, k2, sm4, sm_res, above3);
  const uint32_t kstar = (pre21 << 10) | b3;
  const int ties = k2 - above3;  // keys equal to K* to keep, lowest positions first

  // Walk the staged entries in position order.
  constexpr int E = 4;
  int run_sel = 0, run_tie = 0;
  for (int base = 0; base < n_st; base += kSelThreads * E) {
    u32x2 ent[E];
    int n_eq = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int gi = base + t * E + i;
      ent[i] = (gi < n_st) ? staged(gi) : u32x2{0u, 0u};
      n_eq += (gi < n_st) && (ent[i][0] == kstar);
    }
    int tot_eq;
    int tie_rank = run_tie + block_exclusive_scan(n_eq, sm4, tot_eq);
    bool sel[E];
    int n_sel = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int gi = base + t * E + i;
      bool s = false;
      if (gi < n_st) {
        if (ent[i][0] > kstar) s = true;
        else if (ent[i][0] == kstar) s = (tie_rank++ < ties);
      }
      sel[i] = s;
      n_sel += s;
    }
    int tot_sel;
    int oi = run_sel + block_exclusive_scan(n_sel, sm4, tot_sel);
    const int cap = min(k_eff, a.max_k);
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (sel[i] && oi < cap) {
        const int pos = (int)ent[i][1];
        a.sel_pos[(size_t)b * a.max_k + oi] = pos;
        if (a.sel_slot)
          a.sel_slot[(size_t)b * a.max_k + oi] =
              a.page_table[(size_t)b * a.max_pages + pos / a.page_size] * a.page_size +
              pos % a.page_size;
        ++oi;
      }
    run_sel += tot_sel;
    run_tie += tot_eq;
  }
  if (t == 0) {
    a.sel_count[b] = run_sel;
    atomicExch(&a.ws.done[b], 0u);
  }
}

}  // namespace vg
