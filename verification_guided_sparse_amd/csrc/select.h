// select.h -- score aggregation and exact top-k selection.
//
// Scores map to order-preserving 32-bit keys (larger score <-> larger key;
// -0.0 is folded onto +0.0).  The k-th largest key K* is found by a radix
// select over key bits [20,32) / [10,20) / [0,10), every pass spread over
// chunks of 2048 positions (one workgroup each):
//
//   pass 1  LDS histogram of bits [20,32) per chunk, merged into the
//           sequence's global histogram with atomics (optionally fused with
//           the aggregation that produces the scores).  Also clears the
//           bits [10,20) histogram pass 2 fills.
//   pass 2  each chunk finds the bin b1 holding K*, counts its entries above
//           b1, stages its candidates (bin == b1) in position order and adds
//           their bits [10,20) to a second global histogram.
//   pass 3  each chunk finds b2 from the second histogram, resolves the last
//           10 bits on the (few) candidates, derives from the candidate list
//           how many entries every earlier chunk selects -- hence its own
//           output offset -- and writes its selected positions ascending
//           (keys > K*, then keys == K* lowest position first) with their
//           page-size-1 slots.  Chunk 0 clears the first histogram.
//
// Workgroups hand data to one another only across kernel boundaries; both
// histograms are zero between calls.
#pragma once

#include "vg_device.h"

namespace vg {

constexpr int kSelThreads = 256;
constexpr int kChunk = 2048;                   // positions per pass workgroup
constexpr int kPerThread = kChunk / kSelThreads;  // 8 consecutive positions per thread
constexpr int kBins1 = 4096;                   // key bits [20, 32)
constexpr int kBins23 = 1024;                  // key bits [10, 20), then [0, 10)
constexpr int kMaxChunks = 1024;               // max_prefix <= 2^21
constexpr int kCandCache = 12288;              // candidates a pass-3 workgroup keeps in LDS

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workspace of one selection (per sequence b):
//   hist1  [B][kBins1]  u32   bits [20,32), zero between calls
//   hist2  [B][kBins23] u32   bits [10,20) of the candidates, zero between calls
//   state  [B][4]       i32   b1, entries above bin b1 (written by pass 2)
//   above  [B][kMaxChunks] i32  per chunk: entries above bin b1
//   ncand  [B][kMaxChunks] i32  per chunk: candidates (bin == b1)
//   cand   [B][max_prefix] u32x2 (key, position), chunk w at offset w * kChunk
struct SelWs {
  uint32_t *hist1;
  uint32_t *hist2;
  int32_t *state;
  int32_t *above;
  int32_t *ncand;
  u32x2 *cand;
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
    // rows (t, h) of src in order; batches of 8 rows whose loads are in flight together
    const int nrow = a.src_rows * a.src_heads;
    const float *base = a.src + (size_t)b * nrow * a.max_prefix;
    if (vec) {
      constexpr int U = 8;
      for (int r0 = 0; r0 < nrow; r0 += U) {
        f32x4 v[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (r0 + u < nrow) {
            const float *row = base + (size_t)(r0 + u) * a.max_prefix + j0;
            v[u][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row));
            v[u][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + 4));
          } else {
            v[u][0] = v[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[i] += v[u][0][i];
            sc[4 + i] += v[u][1][i];
          }
      }
    } else {
      for (int r = 0; r < nrow; ++r) {
        const float *row = base + (size_t)r * a.max_prefix;
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

  if (w == 0) {  // pass 2 of this call fills hist2: start it from zero
    uint32_t *h2 = a.ws.hist2 + (size_t)b * kBins23;
    for (int i = t; i < kBins23; i += kSelThreads) h2[i] = 0u;
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (j0 + i < P) atomicAdd(&lh[score_key(sc[i]) >> 20], 1u);
  __syncthreads();
  uint32_t *gh = a.ws.hist1 + (size_t)b * kBins1;
  for (int i = t; i < kBins1; i += kSelThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Load a sequence's bits [20,32) histogram into LDS (16 bins per thread, four
// 16-byte loads in flight together) and find the bin of the k-th largest key.
__device__ __forceinline__ uint32_t load_hist_find_b1(const uint32_t *gh, uint32_t *lh, int k_eff,
                                                      int *sm4, int *sm_res, int &above1) {
  const int t = threadIdx.x;
  const u32x4 *g4 = reinterpret_cast<const u32x4 *>(gh) + 4 * t;
  u32x4 h4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h4[i] = g4[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4 *>(lh)[4 * t + i] = h4[i];
  __syncthreads();
  return (uint32_t)find_bin(lh, kBins1, k_eff, sm4, sm_res, above1);
}

// Pass 2.  grid (nchunks, B).
__global__ __launch_bounds__(kSelThreads) void select_pass2_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins1];
  __shared__ int sm4[4];
  __shared__ int sm_res[2];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = a.prefix_len[b];
  const int k_eff = min(a.k[b], P);
  const int nch = (P + kChunk - 1) / kChunk;
  if (w >= nch) return;
  const int j0 = w * kChunk + t * kPerThread;
  const float *srow = a.scores + (size_t)b * a.max_prefix;
  float sv[kPerThread];  // issued before the histogram work so the loads overlap it
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) sv[i] = (j0 + i < P) ? srow[j0 + i] : 0.f;
  uint32_t b1 = 0xffffffffu;  // k_eff == 0: nothing above, no candidates
  int above1 = 0;
  if (k_eff > 0) b1 = load_hist_find_b1(a.ws.hist1 + (size_t)b * kBins1, lh, k_eff, sm4, sm_res, above1);
  if (w == 0 && t == 0) {
    a.ws.state[4 * b + 0] = (int)b1;
    a.ws.state[4 * b + 1] = above1;
  }
  for (int i = t; i < kBins23; i += kSelThreads) lh[i] = 0u;  // candidates' bits [10,20)
  __syncthreads();
  uint32_t key[kPerThread];
  int n_above = 0, n_cand = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    key[i] = (j0 + i < P) ? score_key(sv[i]) : 0u;
    const bool in = (j0 + i < P) && (k_eff > 0);
    n_above += in && ((key[i] >> 20) > b1);
    const bool cand = in && ((key[i] >> 20) == b1);
    n_cand += cand;
    if (cand) atomicAdd(&lh[(key[i] >> 10) & 1023u], 1u);
  }
  int tot_above, tot_cand;
  block_exclusive_scan(n_above, sm4, tot_above);
  int off = block_exclusive_scan(n_cand, sm4, tot_cand);
  u32x2 *cst = a.ws.cand + (size_t)b * a.max_prefix + (size_t)w * kChunk;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if ((j0 + i < P) && (k_eff > 0) && ((key[i] >> 20) == b1)) cst[off++] = u32x2{key[i], (uint32_t)(j0 + i)};
  if (t == 0) {
    a.ws.above[(size_t)b * kMaxChunks + w] = tot_above;
    a.ws.ncand[(size_t)b * kMaxChunks + w] = tot_cand;
  }
  uint32_t *h2 = a.ws.hist2 + (size_t)b * kBins23;
  for (int i = t; i < kBins23; i += kSelThreads)
    if (lh[i]) atomicAdd(&h2[i], lh[i]);
}

// Pass 3.  grid (nchunks, B).
__global__ __launch_bounds__(kSelThreads) void select_pass3_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins23];
  __shared__ int csum[kMaxChunks + 1];   // candidate offsets per chunk
  __shared__ int nsel[kMaxChunks];       // entries each chunk selects
  __shared__ int neq[kMaxChunks];        // candidates equal to K* per chunk
  __shared__ u32x2 cache[kCandCache];
  __shared__ int sm4[4];
  __shared__ int sm_res[2];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = a.prefix_len[b];
  const int k_eff = min(a.k[b], P);
  const int nch = (P + kChunk - 1) / kChunk;
  if (P <= 0) {
    if (w == 0 && t == 0) a.sel_count[b] = 0;
    return;
  }
  if (w >= nch) return;
  const int j0 = w * kChunk + t * kPerThread;
  const float *srow = a.scores + (size_t)b * a.max_prefix;
  float sv[kPerThread];  // issued first: independent of everything below
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) sv[i] = (j0 + i < P) ? srow[j0 + i] : 0.f;
  if (w == 0) {  // every reader of hist1 has finished (pass 2): clear it for the next call
    u32x4 *g4 = reinterpret_cast<u32x4 *>(a.ws.hist1 + (size_t)b * kBins1) + 4 * t;
#pragma unroll
    for (int i = 0; i < 4; ++i) g4[i] = u32x4{0u, 0u, 0u, 0u};
    if (t == 0) a.sel_count[b] = k_eff;
  }
  if (k_eff <= 0) return;
  const uint32_t b1 = (uint32_t)a.ws.state[4 * b + 0];
  const int above1 = a.ws.state[4 * b + 1];
  // hist2 (4 bins per thread) and the per-chunk counts, loaded together
  const u32x4 h4 = reinterpret_cast<const u32x4 *>(a.ws.hist2 + (size_t)b * kBins23)[t];
  const int per = (nch + kSelThreads - 1) / kSelThreads;  // <= 4
  int ab[4], nc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t * per + i;
    const bool ok = i < per && c < nch;
    ab[i] = ok ? a.ws.above[(size_t)b * kMaxChunks + c] : 0;
    nc[i] = ok ? a.ws.ncand[(size_t)b * kMaxChunks + c] : 0;
  }
  reinterpret_cast<u32x4 *>(lh)[t] = h4;
  {
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) local += nc[i];
    int tot;
    int run = block_exclusive_scan(local, sm4, tot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t * per + i;
      if (i < per && c < nch) {
        csum[c] = run;
        run += nc[i];
        nsel[c] = 0;
        neq[c] = 0;
      }
    }
    if (t == 0) csum[nch] = tot;
  }
  __syncthreads();
  const int k1 = k_eff - above1;  // >= 1: rank of K* inside bin b1
  int above2;
  const uint32_t b2 = (uint32_t)find_bin(lh, kBins23, k1, sm4, sm_res, above2);
  const int k2 = k1 - above2;
  const uint32_t pre22 = (b1 << 10) | b2;
  const int n_c = csum[nch];
  const u32x2 *cand = a.ws.cand + (size_t)b * a.max_prefix;
  auto cand_global = [&](int gi) -> u32x2 {  // candidate number gi, chunk order
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (csum[mid] <= gi) lo = mid; else hi = mid - 1;
    }
    return cand[(size_t)lo * kChunk + (gi - csum[lo])];
  };
  const bool cached = n_c <= kCandCache;
  if (cached) {
    constexpr int U = 8;
    for (int base = 0; base < n_c; base += kSelThreads * U) {
      u32x2 v[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int gi = base + i * kSelThreads + t;
        v[i] = gi < n_c ? cand_global(gi) : u32x2{0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int gi = base + i * kSelThreads + t;
        if (gi < n_c) cache[gi] = v[i];
      }
    }
  }
  for (int i = t; i < kBins23; i += kSelThreads) lh[i] = 0u;
  __syncthreads();
  auto candidate = [&](int gi) -> u32x2 { return cached ? cache[gi] : cand_global(gi); };
  // bits [0, 10) among candidates sharing the 22-bit prefix of K*
  for (int gi = t; gi < n_c; gi += kSelThreads) {
    const u32x2 e = candidate(gi);
    if ((e[0] >> 10) == pre22) atomicAdd(&lh[e[0] & 1023u], 1u);
  }
  __syncthreads();
  int above3;
  const uint32_t b3 = (uint32_t)find_bin(lh, kBins23, k2, sm4, sm_res, above3);
  const uint32_t kstar = (pre22 << 10) | b3;
  const int ties = k2 - above3;  // entries equal to K* to keep, lowest positions first
  // per chunk: candidates above K* and candidates equal to K*
  for (int gi = t; gi < n_c; gi += kSelThreads) {
    const u32x2 e = candidate(gi);
    const int c = (int)(e[1] / kChunk);
    if (e[0] > kstar) atomicAdd(&nsel[c], 1);
    else if (e[0] == kstar) atomicAdd(&neq[c], 1);
  }
  __syncthreads();
  // Per chunk c: taken_c = ties left after the chunks before it, capped by its
  // own equal candidates; selected_c = above_c + (candidates > K*) + taken_c.
  // The thread owning chunk w publishes the exclusive prefixes at w.
  int eq_before, sel_before;
  {
    int eqv[4], eq_local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t * per + i;
      eqv[i] = (i < per && c < nch) ? neq[c] : 0;
      eq_local += eqv[i];
    }
    int tot;
    int eq_run = block_exclusive_scan(eq_local, sm4, tot);
    int selv[4], sel_local = 0, eq_at[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t * per + i;
      eq_at[i] = eq_run;
      selv[i] = 0;
      if (i < per && c < nch) {
        const int taken = max(0, min(eqv[i], ties - eq_run));
        selv[i] = ab[i] + nsel[c] + taken;
      }
      sel_local += selv[i];
      eq_run += eqv[i];
    }
    int sel_run = block_exclusive_scan(sel_local, sm4, tot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t * per + i;
      if (i < per && c == w) {
        sm_res[0] = sel_run;
        sm_res[1] = eq_at[i];
      }
      sel_run += selv[i];
    }
    __syncthreads();
    sel_before = sm_res[0];
    eq_before = sm_res[1];
    __syncthreads();
  }
  // Select this chunk's entries in position order.
  uint32_t key[kPerThread];
  int n_eq = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    key[i] = (j0 + i < P) ? score_key(sv[i]) : 0u;
    n_eq += (j0 + i < P) && (key[i] == kstar);
  }
  int tot_eq;
  int tie_rank = eq_before + block_exclusive_scan(n_eq, sm4, tot_eq);
  bool sel[kPerThread];
  int n_sel = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    bool s = false;
    if (j0 + i < P) {
      if (key[i] > kstar) s = true;
      else if (key[i] == kstar) s = (tie_rank++ < ties);
    }
    sel[i] = s;
    n_sel += s;
  }
  int tot_sel;
  int oi = sel_before + block_exclusive_scan(n_sel, sm4, tot_sel);
  const int cap = min(k_eff, a.max_k);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (sel[i] && oi < cap) {
      const int pos = j0 + i;
      a.sel_pos[(size_t)b * a.max_k + oi] = pos;
      if (a.sel_slot)
        a.sel_slot[(size_t)b * a.max_k + oi] =
            a.page_table[(size_t)b * a.max_pages + pos / a.page_size] * a.page_size + pos % a.page_size;
      ++oi;
    }
}

}  // namespace vg
