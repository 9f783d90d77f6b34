// select.h -- score aggregation and exact top-k selection.
//
// Scores map to order-preserving 32-bit keys (larger score <-> larger key;
// -0.0 is folded onto +0.0).  The k-th largest key K* is found by a radix
// select over key bits [20,32) / [10,20) / [0,10), passes 2 and 3 spread
// over chunks of 2048 positions:
//
//   pass 1  (one workgroup per 512 positions) LDS histogram of bits [20,32),
//           merged into the sequence's global histogram with atomics
//           (optionally fused with the aggregation that produces the scores,
//           a latency-bound stream of the export that wants many workgroups).
//           Also clears the bits [10,20) histogram pass 2 fills.
//   pass 2  (one workgroup per chunk) finds the bin b1 holding K*, counts the
//           chunk's entries above b1, stages its candidates (bin == b1) in
//           position order and adds their bits [10,20) to a second global
//           histogram.
//   pass 3  (one workgroup per chunk) finds b2 from the second histogram,
//           resolves the last 10 bits on the candidates (a fixed group of
//           threads per chunk reads that chunk's candidates), counts per chunk
//           the candidates above and equal to K*, derives its own output offset
//           from those counts, and writes its selected positions ascending
//           (keys > K*, then keys == K* lowest position first) with their
//           page-size-1 slots.  Chunk 0 clears the first histogram.
//
// Ties at K* are taken in position order, so the ties taken before a point
// are min(ties, equal keys before it): one scan of (greater, equal) counts
// gives every output offset.
//
// Workgroups hand data to one another only across kernel boundaries; both
// histograms are zero between calls.
#pragma once

#include "vg_device.h"

namespace vg {

constexpr int kSelThreads = 256;
constexpr int kChunk = 2048;                   // positions per pass-2/3 workgroup
constexpr int kPerThread = kChunk / kSelThreads;  // 8 consecutive positions per thread
constexpr int kBins1 = 4096;                   // key bits [20, 32)
constexpr int kBins23 = 1024;                  // key bits [10, 20), then [0, 10)
constexpr int kMaxChunks = 1024;               // max_prefix <= 2^21
constexpr int kCandCache = 12288;              // candidates a pass-3 workgroup keeps in LDS
constexpr int kTieList = 1024;                 // pass 3 fast path: candidates sharing K*'s 22-bit prefix

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

// Prefix length and selection size of sequence b, clamped to what the
// buffers were sized for: 0 <= P <= max_prefix and 0 <= kk <= min(P, max_k).
__device__ __forceinline__ int sel_prefix(const SelArgs &a, int b) {
  return min(max(a.prefix_len[b], 0), a.max_prefix);
}
__device__ __forceinline__ int sel_k(const SelArgs &a, int b, int P) {
  return min(min(max(a.k[b], 0), P), a.max_k);
}

// Rank search over a histogram held in registers: thread t holds the PER bins
// [nbins - PER (t + 1), nbins - PER t) in descending order (h[0] = the
// highest).  Finds the bin holding the k-th largest key (1 <= k <= total) and,
// in `above`, the number of keys in higher bins.  Block-wide; every thread gets
// the result.  `res` (2 ints of LDS) must not be shared with a call whose
// results are still being read.
template <int PER>
__device__ __forceinline__ int find_bin_regs(const uint32_t (&h)[PER], int nbins, int k, int *sm4,
                                             int *res, int &above, int *count = nullptr) {
  const int t = threadIdx.x;
  const int top = nbins - PER * t;
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += (int)h[i];
  if (t == 0) {
    res[0] = 0;
    res[1] = 0;
    if (count) res[2] = 0;
  }
  int total;
  const int pre = block_exclusive_scan(local, sm4, total);  // its barriers order the reset above
  if (pre < k && k <= pre + local) {
    int run = pre;
    bool done = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = (int)h[i];
      if (!done && k <= run + c) {
        res[0] = top - 1 - i;
        res[1] = run;
        if (count) res[2] = c;
        done = true;
      }
      run += c;
    }
  }
  __syncthreads();
  above = res[1];
  if (count) *count = res[2];
  return res[0];
}

// Thread t's PER descending bins of a global (or LDS) histogram of nbins.
template <int PER>
__device__ __forceinline__ void load_bins_desc(const uint32_t *hist, int nbins, uint32_t (&h)[PER]) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(hist + nbins - PER * (threadIdx.x + 1));
  u32x4 v[PER / 4];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) v[i] = src[i];
#pragma unroll
  for (int i = 0; i < PER; ++i) h[i] = v[(PER - 1 - i) / 4][(PER - 1 - i) % 4];
}

// Pass 1.  grid (ceil(max_prefix / kP1Block), B), kP1Threads threads (kP1Per
// consecutive positions each).  AGG: compute scores from src and write them.
// HIST: add the block's bits [20,32) histogram to the global one.
// Aggregation is a latency-bound stream of src rows: the bytes in flight are
// P x kP1Rows floats whatever the block size, so the rows of a batch are
// many, and the blocks small enough that every CU has one.
constexpr int kP1Threads = 256;
constexpr int kP1Per = 2;
constexpr int kP1Block = kP1Threads * kP1Per;  // 512 positions
constexpr int kP1Rows = 32;                    // src rows whose loads are in flight together
typedef float p1vec __attribute__((ext_vector_type(kP1Per)));

template <bool AGG, bool HIST>
__global__ __launch_bounds__(kP1Threads) void select_pass1_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins1];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = sel_prefix(a, b);
  if (w >= (P + kP1Block - 1) / kP1Block) return;
  if (HIST) {
    for (int i = t; i < kBins1 / 4; i += kP1Threads) reinterpret_cast<u32x4 *>(lh)[i] = u32x4{0u, 0u, 0u, 0u};
  }
  const int j0 = w * kP1Block + t * kP1Per;
  float sc[kP1Per];
#pragma unroll
  for (int i = 0; i < kP1Per; ++i) sc[i] = 0.f;
  if (AGG) {
    const bool vec = ((a.max_prefix % kP1Per) == 0) && (j0 + kP1Per <= P);
    // rows (t, h) of src in order, added in that order; batches of kP1Rows
    // rows whose loads are in flight together
    const int nrow = a.src_rows * a.src_heads;
    const float *base = a.src + (size_t)b * nrow * a.max_prefix;
    if (vec) {
      for (int r0 = 0; r0 < nrow; r0 += kP1Rows) {
        p1vec v[kP1Rows];
#pragma unroll
        for (int u = 0; u < kP1Rows; ++u)
          v[u] = (r0 + u < nrow) ? __builtin_nontemporal_load(reinterpret_cast<const p1vec *>(
                                       base + (size_t)(r0 + u) * a.max_prefix + j0))
                                 : p1vec{};
#pragma unroll
        for (int u = 0; u < kP1Rows; ++u)
#pragma unroll
          for (int i = 0; i < kP1Per; ++i) sc[i] += v[u][i];
      }
    } else {
      for (int r = 0; r < nrow; ++r) {
        const float *row = base + (size_t)r * a.max_prefix;
#pragma unroll
        for (int i = 0; i < kP1Per; ++i)
          if (j0 + i < P) sc[i] += row[j0 + i];
      }
    }
    float *dst = a.scores_out + (size_t)b * a.max_prefix;
    if (vec) {
      p1vec o;
#pragma unroll
      for (int i = 0; i < kP1Per; ++i) o[i] = sc[i];
      *reinterpret_cast<p1vec *>(dst + j0) = o;
    } else {
#pragma unroll
      for (int i = 0; i < kP1Per; ++i)
        if (j0 + i < P) dst[j0 + i] = sc[i];
    }
  } else {
    const float *srow = a.scores + (size_t)b * a.max_prefix;
#pragma unroll
    for (int i = 0; i < kP1Per; ++i) sc[i] = (j0 + i < P) ? srow[j0 + i] : 0.f;
  }
  if (!HIST) return;

  if (w == 0) {  // pass 2 of this call fills hist2: start it from zero
    uint32_t *h2 = a.ws.hist2 + (size_t)b * kBins23;
    for (int i = t; i < kBins23; i += kP1Threads) h2[i] = 0u;
  }
  __syncthreads();  // the LDS histogram is clear
#pragma unroll
  for (int i = 0; i < kP1Per; ++i)
    if (j0 + i < P) atomicAdd(&lh[score_key(sc[i]) >> 20], 1u);
  __syncthreads();
  // consecutive lanes take consecutive bins: one atomic instruction then
  // touches as few cache lines as possible
  uint32_t *gh = a.ws.hist1 + (size_t)b * kBins1;
  for (int i = t; i < kBins1; i += kP1Threads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Pass 2.  grid (nchunks, B).
__global__ __launch_bounds__(kSelThreads) void select_pass2_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins23];
  __shared__ int sm4[4];
  __shared__ int sm_res[2];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = sel_prefix(a, b);
  const int k_eff = sel_k(a, b, P);
  const int nch = (P + kChunk - 1) / kChunk;
  if (w >= nch) return;
  const int j0 = w * kChunk + t * kPerThread;
  const float *srow = a.scores + (size_t)b * a.max_prefix;
  float sv[kPerThread];  // issued first: independent of everything below
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) sv[i] = (j0 + i < P) ? srow[j0 + i] : 0.f;
  reinterpret_cast<u32x4 *>(lh)[t] = u32x4{0u, 0u, 0u, 0u};  // candidates' bits [10,20)
  uint32_t b1 = 0xffffffffu;  // k_eff == 0: nothing above, no candidates
  int above1 = 0;
  if (k_eff > 0) {
    uint32_t h[16];
    load_bins_desc<16>(a.ws.hist1 + (size_t)b * kBins1, kBins1, h);
    b1 = (uint32_t)find_bin_regs<16>(h, kBins1, k_eff, sm4, sm_res, above1);  // also orders the clear
  } else {
    __syncthreads();
  }
  if (w == 0 && t == 0) {
    a.ws.state[4 * b + 0] = (int)b1;
    a.ws.state[4 * b + 1] = above1;
  }
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
  // one scan of both counts (each <= 2048)
  int tot;
  int off = block_exclusive_scan(n_above | (n_cand << 16), sm4, tot);
  const int tot_above = tot & 0xffff, tot_cand = tot >> 16;
  off >>= 16;
  u32x2 *cst = a.ws.cand + (size_t)b * a.max_prefix + (size_t)w * kChunk;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if ((j0 + i < P) && (k_eff > 0) && ((key[i] >> 20) == b1)) cst[off++] = u32x2{key[i], (uint32_t)(j0 + i)};
  if (t == 0) {
    a.ws.above[(size_t)b * kMaxChunks + w] = tot_above;
    a.ws.ncand[(size_t)b * kMaxChunks + w] = tot_cand;
  }
  // the scan's barriers ordered the LDS histogram atomics before these reads;
  // consecutive lanes take consecutive bins
  uint32_t *h2 = a.ws.hist2 + (size_t)b * kBins23;
  for (int i = t; i < kBins23; i += kSelThreads)
    if (lh[i]) atomicAdd(&h2[i], lh[i]);
}

// Pass 3.  grid (nchunks, B).
__global__ __launch_bounds__(kSelThreads) void select_pass3_kernel(SelArgs a) {
  __shared__ uint32_t lh[kBins23];
  __shared__ int csum[kMaxChunks + 1];  // candidate offsets per chunk
  __shared__ int cgt[kMaxChunks];       // per chunk: candidates above K*
  __shared__ int ceq[kMaxChunks];       // per chunk: candidates equal to K*
  __shared__ u32x2 cache[kCandCache];
  __shared__ uint32_t tie[kTieList];   // fast path: candidates sharing K*'s 22-bit prefix
  __shared__ int tie_n;
  __shared__ int sm4[4];
  __shared__ int sm_res[8];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int P = sel_prefix(a, b);
  const int k_eff = sel_k(a, b, P);
  const int nch = (P + kChunk - 1) / kChunk;
  if (P <= 0) {
    if (w == 0 && t == 0) a.sel_count[b] = 0;
    return;
  }
  if (w >= nch) return;
  // ---- loads that depend on nothing else, issued first
  const int j0 = w * kChunk + t * kPerThread;
  const float *srow = a.scores + (size_t)b * a.max_prefix;
  float sv[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) sv[i] = (j0 + i < P) ? srow[j0 + i] : 0.f;
  // page ids of this thread's 8 positions, loaded now: a load among the output
  // stores at the end would make each store wait for the ones before it
  // (loads and stores retire in order on one counter)
  int page[kPerThread] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool one_page = (a.page_size & 7) == 0;  // then the 8 positions share a page
  if (a.sel_slot) {
    const int32_t *prow = a.page_table + (size_t)b * a.max_pages;
    if (one_page) {
      const int pg = j0 < P ? prow[j0 / a.page_size] : 0;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) page[i] = pg;
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) page[i] = j0 + i < P ? prow[(j0 + i) / a.page_size] : 0;
    }
  }
  if (w == 0) {  // every reader of hist1 has finished (pass 2): clear it for the next call
    u32x4 *g4 = reinterpret_cast<u32x4 *>(a.ws.hist1 + (size_t)b * kBins1) + 4 * t;
#pragma unroll
    for (int i = 0; i < 4; ++i) g4[i] = u32x4{0u, 0u, 0u, 0u};
    if (t == 0) a.sel_count[b] = k_eff;
  }
  if (k_eff <= 0) return;
  const uint32_t b1 = (uint32_t)a.ws.state[4 * b + 0];
  const int above1 = a.ws.state[4 * b + 1];
  uint32_t h2[4];
  load_bins_desc<4>(a.ws.hist2 + (size_t)b * kBins23, kBins23, h2);
  // per-chunk counts: thread t owns chunks t * per + i
  const int per = (nch + kSelThreads - 1) / kSelThreads;  // <= 4
  int ab[4], nc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t * per + i;
    const bool ok = i < per && c < nch;
    ab[i] = ok ? a.ws.above[(size_t)b * kMaxChunks + c] : 0;
    nc[i] = ok ? a.ws.ncand[(size_t)b * kMaxChunks + c] : 0;
  }
  reinterpret_cast<u32x4 *>(lh)[t] = u32x4{0u, 0u, 0u, 0u};  // bits [0,10) of the candidates
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
      }
    }
    if (t == 0) csum[nch] = tot;
  }
  const int k1 = k_eff - above1;  // >= 1: rank of K* inside bin b1
  int above2;
  int n_b2;  // candidates sharing K*'s 22-bit prefix
  if (t == 0) tie_n = 0;  // ordered before its atomics by find_bin_regs' barriers
  const uint32_t b2 =
      (uint32_t)find_bin_regs<4>(h2, kBins23, k1, sm4, sm_res, above2, &n_b2);  // csum visible after
  const int k2 = k1 - above2;
  const uint32_t pre22 = (b1 << 10) | b2;
  const int n_c = csum[nch];
  const u32x2 *cand = a.ws.cand + (size_t)b * a.max_prefix;
  // Candidates of chunk c are read by a fixed group of tpc consecutive threads
  // (tpc = 256 / nch rounded down to a power of two, at most a wave; for
  // nch > 256 every thread takes chunks t, t + 256, ...): no search for a
  // candidate's chunk.
  int tpc = 1;
  while (tpc < kWave && tpc * 2 * nch <= kSelThreads) tpc *= 2;
  const int sub = t % tpc, c_first = t / tpc, c_step = kSelThreads / tpc;
  uint32_t kstar;
  int ties;  // entries equal to K* to keep, lowest positions first
  if (n_b2 <= kTieList) {
    // Fast path: one pass over the candidates (keys only, from global) counts
    // per chunk those above K*'s 22-bit prefix, and gathers the few sharing
    // it (their low 10 bits and chunk) into LDS with their bit histogram.
    // K* then follows from that histogram, and the gathered candidates
    // complete the per-chunk counts above and equal to K*.
    const uint32_t *ckey = reinterpret_cast<const uint32_t *>(cand);
    for (int c = c_first; c < nch; c += c_step) {
      const int n = csum[c + 1] - csum[c];
      int gt = 0;
      for (int i0 = sub; i0 < n; i0 += 8 * tpc) {
        uint32_t kq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kq[u] = i0 + u * tpc < n ? ckey[2 * ((size_t)c * kChunk + i0 + u * tpc)] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (i0 + u * tpc < n) {
            const uint32_t hi = kq[u] >> 10;
            gt += hi > pre22;
            if (hi == pre22) {
              atomicAdd(&lh[kq[u] & 1023u], 1u);
              const int q = atomicAdd(&tie_n, 1);  // < n_b2 <= kTieList
              if (q < kTieList) tie[q] = (kq[u] & 1023u) | ((uint32_t)c << 10);
            }
          }
        }
      }
      for (int o = 1; o < tpc; o <<= 1) gt += __shfl_xor(gt, o);
      if (sub == 0) {
        cgt[c] = gt;
        ceq[c] = 0;
      }
    }
    __syncthreads();
    uint32_t h3[4];
    load_bins_desc<4>(lh, kBins23, h3);
    int above3;
    const uint32_t b3 = (uint32_t)find_bin_regs<4>(h3, kBins23, k2, sm4, sm_res + 3, above3);
    kstar = (pre22 << 10) | b3;
    ties = k2 - above3;
    for (int i = t; i < min(n_b2, kTieList); i += kSelThreads) {
      const uint32_t low = tie[i] & 1023u, c = tie[i] >> 10;
      if (low > b3) atomicAdd(&cgt[c], 1);
      else if (low == b3) atomicAdd(&ceq[c], 1);
    }
    __syncthreads();
  } else {
  const bool cached = n_c <= kCandCache;
  if (cached) {
    for (int c = c_first; c < nch; c += c_step) {
      const int n = csum[c + 1] - csum[c];
      for (int i0 = sub; i0 < n; i0 += tpc * 8) {
        u32x2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * tpc;
          v[u] = i < n ? cand[(size_t)c * kChunk + i] : u32x2{0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * tpc;
          if (i < n) cache[csum[c] + i] = v[u];
        }
      }
    }
    __syncthreads();
  }
  auto candidate = [&](int c, int i) -> u32x2 {
    return cached ? cache[csum[c] + i] : cand[(size_t)c * kChunk + i];
  };
  // bits [0, 10) among candidates sharing the 22-bit prefix of K* (reads in
  // batches of 4, all in flight together)
  for (int c = c_first; c < nch; c += c_step) {
    const int n = csum[c + 1] - csum[c];
    for (int i0 = sub; i0 < n; i0 += 4 * tpc) {
      uint32_t kq[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kq[u] = i0 + u * tpc < n ? candidate(c, i0 + u * tpc)[0] : 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * tpc < n && (kq[u] >> 10) == pre22) atomicAdd(&lh[kq[u] & 1023u], 1u);
    }
  }
  __syncthreads();
  uint32_t h3[4];
  load_bins_desc<4>(lh, kBins23, h3);
  int above3;
  const uint32_t b3 = (uint32_t)find_bin_regs<4>(h3, kBins23, k2, sm4, sm_res + 3, above3);
  kstar = (pre22 << 10) | b3;
  ties = k2 - above3;
  // per chunk: candidates above and equal to K*, summed over the chunk's group
  for (int c = c_first; c < nch; c += c_step) {
    const int n = csum[c + 1] - csum[c];
    int gt = 0, eq = 0;
    for (int i0 = sub; i0 < n; i0 += 4 * tpc) {
      uint32_t kq[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kq[u] = i0 + u * tpc < n ? candidate(c, i0 + u * tpc)[0] : 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gt += (i0 + u * tpc < n) && kq[u] > kstar;
        eq += (i0 + u * tpc < n) && kq[u] == kstar;
      }
    }
    // the group is tpc consecutive lanes of one wave (tpc <= 64 divides 64)
    for (int o = 1; o < tpc; o <<= 1) {
      gt += __shfl_xor(gt, o);
      eq += __shfl_xor(eq, o);
    }
    if (sub == 0) {
      cgt[c] = gt;
      ceq[c] = eq;
    }
  }
  __syncthreads();
  }
  // Output offset of chunk w: entries above K* in earlier chunks plus the ties
  // they take, min(ties, equal keys in earlier chunks).
  int sel_before, eq_before;
  {
    int gv[4], ev[4], g_local = 0, e_local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t * per + i;
      const bool ok = i < per && c < nch;
      gv[i] = ok ? ab[i] + cgt[c] : 0;
      ev[i] = ok ? ceq[c] : 0;
      g_local += gv[i];
      e_local += ev[i];
    }
    int gt_tot, eq_tot;
    int g_run = block_exclusive_scan(g_local, sm4, gt_tot);
    int e_run = block_exclusive_scan(e_local, sm4, eq_tot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t * per + i;
      if (i < per && c == w) {
        sm_res[6] = g_run + min(ties, e_run);
        sm_res[7] = e_run;
      }
      g_run += gv[i];
      e_run += ev[i];
    }
    __syncthreads();
    sel_before = sm_res[6];
    eq_before = sm_res[7];
  }
  // Select this chunk's entries in position order: one scan of the packed
  // (greater, equal) counts (each <= 2048) gives every thread's offset.
  uint32_t key[kPerThread];
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    key[i] = (j0 + i < P) ? score_key(sv[i]) : 0u;
    n_gt += (j0 + i < P) && (key[i] > kstar);
    n_eq += (j0 + i < P) && (key[i] == kstar);
  }
  int tot;
  const int ex = block_exclusive_scan(n_gt | (n_eq << 16), sm4, tot);
  const int gt_before = ex & 0xffff, eq_in = ex >> 16;
  const int tie_budget = max(0, ties - eq_before);  // ties left for this chunk
  int eq_rank = eq_in;
  // rank of this thread's first selected entry inside the chunk
  int li = gt_before + min(tie_budget, eq_in);
  const int n_sel = (tot & 0xffff) + min(tie_budget, tot >> 16);  // the chunk's selections
  // Stage the chunk's selected positions (and their page ids) in LDS in order
  // -- at most 2048; the candidate cache is free again -- then write them out
  // with consecutive lanes on consecutive outputs.
  int *st_pos = reinterpret_cast<int *>(cache);  // its readers finished before the scans above
  int *st_page = st_pos + kChunk;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    bool s = false;
    if (j0 + i < P) {
      if (key[i] > kstar) s = true;
      else if (key[i] == kstar) s = (eq_rank++ < tie_budget);
    }
    if (s) {
      st_pos[li] = j0 + i;
      st_page[li] = page[i];
    }
    li += s;
  }
  __syncthreads();
  const int n_out = min(n_sel, min(k_eff, a.max_k) - sel_before);
  int32_t *pos_row = a.sel_pos + (size_t)b * a.max_k + sel_before;
  int32_t *slot_row = a.sel_slot ? a.sel_slot + (size_t)b * a.max_k + sel_before : nullptr;
  for (int q = t; q < n_out; q += kSelThreads) {
    const int pos = st_pos[q];
    pos_row[q] = pos;
    if (slot_row) slot_row[q] = st_page[q] * a.page_size + pos % a.page_size;
  }
}

}  // namespace vg
