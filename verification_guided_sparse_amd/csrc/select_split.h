// select_split.h -- exact top-k selection (optionally with the score
// aggregation) in two launches, for prefixes of up to kSplitMaxPrefix
// positions.  Both kernels take one workgroup per chunk of 2048 positions of
// each sequence.
//
//   stage    aggregate the chunk's scores from the export (or read them), key
//            them (order-preserving uint32) and histogram the top 12 key bits
//            in LDS.  Write the chunk's (key, position) pairs grouped by bin,
//            highest bin first (`staged`), and per bin the number of the
//            chunk's keys in that bin or above (`cnt_ge`, and every 64th bin
//            of it transposed into `coarse`).
//   resolve  every workgroup finds the sequence's k-th largest key K* by
//            itself, from data that is small and shared by all of them: the
//            bin b1 holding it (the sums over chunks of cnt_ge, searched 64
//            bins at a time: coarse, then the 64-bin window), and K* within
//            b1 from the candidates (bin b1: staged entries cnt_ge[b1 + 1] ..
//            cnt_ge[b1] of every chunk): a histogram of key bits [10, 20)
//            gives the 22-bit bin b2, then either one wave ranks b2's keys
//            (when there are at most 64) or a histogram of bits [0, 10) does.  Then
//            it writes its own chunk's selection: the staged entries above b1,
//            the candidates above K*, and the keys equal to K* that the tie
//            rule gives this chunk (lowest positions first, so earlier chunks
//            take theirs first), in ascending position order at the chunk's
//            offset, with their page-size-1 slots.
//
// No workgroup waits for another inside a kernel; the kernel boundary is the
// only handoff.  The work that depends on one step (K*) is repeated by every
// workgroup, so the chain of dependent steps after the boundary is short:
// three rounds of loads (coarse counts, the window's counts, the candidates)
// and LDS work.  The selected set does not depend on the order of staged
// entries within a bin, so the result is deterministic although the staging
// uses LDS atomics.
//
// Written around three properties of the hardware: a workgroup barrier
// waits for every global load and store the wave has in flight, so the stage
// kernel issues its global writes after its last barrier; a load whose address
// follows a data-dependent branch is not issued together with the others, so
// each round of loads is computed without branches and with wave-uniform
// indices; and a register that a load writes cannot be reused before the load
// returns, so no load writes a half the code never reads.
#pragma once

#include "select.h"

namespace vg {

constexpr int kStageThreads = 1024;
constexpr int kStageWaves = kStageThreads / kWave;
constexpr int kResolveThreads = 512;
constexpr int kResolveWaves = kResolveThreads / kWave;
constexpr int kSplitMaxPrefix = 1 << 17;
constexpr int kSplitMaxChunks = kSplitMaxPrefix / kChunk;  // 64: one wave takes all chunks
constexpr int kCntStride = kBins1 + 8;                     // u16 per chunk row of cnt_ge (16-byte rows)
constexpr int kResolveCache = 6144;                        // candidates kept in LDS
constexpr int kCandPiece = kWave;                          // candidates per read item
constexpr int kItemBatch = 12;                             // candidate items per wave per batch of loads

// Workspace pieces of the two-launch selection (besides SelWs.cand, which
// holds the staged pairs: chunk c at offset c * kChunk).
struct StageWs {
  uint16_t *cnt_ge;  // [B][chunks][kCntStride]: cnt_ge[c][bin] = keys of chunk c in bin or above
  uint16_t *coarse;  // [B][64][kSplitMaxChunks]: cnt_ge[c][64 j] at [j][c]
  int32_t chunks;    // chunk rows per sequence in cnt_ge
};

// Exclusive prefix sum over a block of NW waves; `total` receives the sum.
template <int NW>
__device__ __forceinline__ int block_scan_n(int v, int *sm, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) sm[w] = x;
  __syncthreads();
  int pre = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = sm[i];
    pre += (i < w) ? c : 0;
    total += c;
  }
  __syncthreads();
  return pre + x - v;
}

// Rank search by a block of NW waves over a histogram held PER bins per
// thread, descending (thread t holds bins [nbins - PER (t + 1), nbins - PER t),
// h[0] the highest): the bin holding the k-th largest key (1 <= k <= total),
// the keys in higher bins (`above`) and the bin's own count.  Two barriers;
// `wsum` (NW ints) and `res` (3 ints) of LDS must not be read by a later call
// before its first barrier, so consecutive calls pass different `res`.
template <int NW, int PER>
__device__ __forceinline__ int find_bin_n(const uint32_t (&h)[PER], int nbins, int k, int *wsum, int *res,
                                          int &above, int &count) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += (int)h[i];
  const int x = wave_inclusive_scan(local);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int pre = x - local;
#pragma unroll
  for (int i = 0; i < NW; ++i) pre += (i < w) ? wsum[i] : 0;
  if (pre < k && k <= pre + local) {  // exactly one thread
    int run = pre;
    bool done = false;
    const int top = nbins - PER * t;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = (int)h[i];
      if (!done && k <= run + c) {
        res[0] = top - 1 - i;
        res[1] = run;
        res[2] = c;
        done = true;
      }
      run += c;
    }
  }
  __syncthreads();
  above = res[1];
  count = res[2];
  return res[0];
}

// ---------------------------------------------------------------- stage
// One chunk (w) of sequence b by a block of NT threads, 2048 / NT consecutive
// positions each.  Called by select_stage_kernel (NT = 1024) and by the
// verify call's second kernel next to the combine (NT = 256).  Thread t holds
// the position pairs t, t + NT, t + 2 NT, ... of the chunk, so that each load
// instruction of a wave reads 512 contiguous bytes of an export row.
template <bool AGG, int NT>
__device__ __forceinline__ void stage_block(const SelArgs &a, const StageWs &o, int b, int w) {
  constexpr int PPT = kChunk / NT;  // positions per thread
  constexpr int BPT = kBins1 / NT;  // histogram bins per thread
  constexpr int NW = NT / kWave;
  static_assert(PPT % 2 == 0 && BPT % 4 == 0, "block size");
  __shared__ uint32_t hist[kBins1];  // the histogram, then the counting-sort cursors
  __shared__ u32x2 staged[kChunk];
  __shared__ int wsum[NW];
  const int t = threadIdx.x;
  // loads first, before the length is known (positions below max_prefix are
  // inside every row, and max_prefix is even)
  const int c0 = w * kChunk;
  auto pos_of = [&](int i) { return c0 + 2 * (t + NT * (i / 2)) + (i & 1); };  // position of key i
  const int P = sel_prefix(a, b);
  f32x2 sc[PPT / 2];
#pragma unroll
  for (int i = 0; i < PPT / 2; ++i) sc[i] = f32x2{0.f, 0.f};
  if (AGG) {
    const int nrow = a.src_rows * a.src_heads;
    const float *base = a.src + (size_t)b * nrow * a.max_prefix;
    constexpr int UR = 8;  // rows per batch (rows are summed in order: the same sums at any NT)
    for (int r0 = 0; r0 < nrow; r0 += UR) {
      f32x2 v[UR][PPT / 2];
#pragma unroll
      for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int i = 0; i < PPT / 2; ++i)
          v[u][i] = (pos_of(2 * i) < a.max_prefix && r0 + u < nrow)
                        ? __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(
                              base + (size_t)(r0 + u) * a.max_prefix + pos_of(2 * i)))
                        : f32x2{0.f, 0.f};
#pragma unroll
      for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int i = 0; i < PPT / 2; ++i) sc[i] += v[u][i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PPT / 2; ++i)
      if (pos_of(2 * i) < a.max_prefix)
        sc[i] = *reinterpret_cast<const f32x2 *>(a.scores + (size_t)b * a.max_prefix + pos_of(2 * i));
  }
  const int nch = (P + kChunk - 1) / kChunk;
  if (w >= nch) return;
  uint32_t key[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) key[i] = score_key(sc[i / 2][i % 2]);
#pragma unroll
  for (int i = 0; i < BPT; ++i) hist[t + i * NT] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PPT; ++i)
    if (pos_of(i) < P) atomicAdd(&hist[key[i] >> 20], 1u);
  __syncthreads();
  // cnt_ge: thread t owns bins [4096 - BPT (t + 1), 4096 - BPT t), highest first
  const int top = kBins1 - BPT * t;
  uint32_t hh[BPT], ge[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) hh[i] = hist[top - 1 - i];
  {
    int local = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) local += (int)hh[i];
    int total;
    int run = block_scan_n<NW>(local, wsum, total);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      run += (int)hh[i];
      ge[i] = (uint32_t)run;  // keys in bin top - 1 - i or above
    }
  }
  // counting sort by bin, highest first: the cursor starts at the keys above the bin
#pragma unroll
  for (int i = 0; i < BPT; ++i) hist[top - 1 - i] = ge[i] - hh[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PPT; ++i)
    if (pos_of(i) < P) staged[atomicAdd(&hist[key[i] >> 20], 1u)] = u32x2{key[i], (uint32_t)pos_of(i)};
  __syncthreads();
  // global writes, after the last barrier
  if (AGG) {
    float *dst = a.scores_out + (size_t)b * a.max_prefix;
#pragma unroll
    for (int i = 0; i < PPT / 2; ++i) {
      const int p = pos_of(2 * i);
      if (p + 1 < P) *reinterpret_cast<f32x2 *>(dst + p) = sc[i];
      else if (p < P) dst[p] = sc[i][0];
    }
  }
  uint16_t *row = o.cnt_ge + ((size_t)b * o.chunks + w) * kCntStride;
#pragma unroll
  for (int i = 0; i < BPT; i += 4)  // bins top - 4 - i .. top - 1 - i, lowest first
    *reinterpret_cast<u32x2 *>(row + top - 4 - i) =
        u32x2{ge[i + 3] | (ge[i + 2] << 16), ge[i + 1] | (ge[i] << 16)};
  if (t == 0) row[kBins1] = 0;
  constexpr int TPC = 64 / BPT;  // threads per 64 bins
  if (t % TPC == TPC - 1) {      // bin 64 j is the lowest of thread NT - 1 - TPC j's bins
    const int j = (NT - 1 - t) / TPC;
    o.coarse[((size_t)b * 64 + j) * kSplitMaxChunks + w] = (uint16_t)ge[BPT - 1];
  }
  const int n = min(P - w * kChunk, kChunk);
  u32x2 *dst = a.ws.cand + (size_t)b * a.max_prefix + (size_t)w * kChunk;
#pragma unroll
  for (int i = 0; i < PPT; i += 2) {
    const int e = PPT * t + i;
    if (e + 1 < n)
      *reinterpret_cast<u32x4 *>(dst + e) = u32x4{staged[e][0], staged[e][1], staged[e + 1][0], staged[e + 1][1]};
    else if (e < n)
      dst[e] = staged[e];
  }
}

template <bool AGG>
__global__ __launch_bounds__(kStageThreads, 2) void select_stage_kernel(SelArgs a, StageWs o) {
  stage_block<AGG, kStageThreads>(a, o, blockIdx.y, blockIdx.x);
}

// ---------------------------------------------------------------- resolve
struct ResolveSmem {
  u32x2 cache[kResolveCache];  // the sequence's candidates, chunk by chunk
  uint32_t h[kBins23];
  int32_t out[kChunk];         // this chunk's selected positions, ascending
  int part[kResolveWaves][kWave];
  int part64[kResolveWaves];
  int g[kSplitMaxChunks + 1];
  int hi[kSplitMaxChunks], lo[kSplitMaxChunks];
  int cand_off[kSplitMaxChunks + 1];
  int gt[kSplitMaxChunks], eq[kSplitMaxChunks];
  uint32_t bm[kChunk / 32];   // this chunk's selected positions
  uint32_t tie[kChunk / 32];  // this chunk's keys equal to K*
  int32_t page[kChunk / kPageSize];
  u32x2 list[kWave];  // the candidates of the second-level bin holding K*, when few
  int meta[8];
};

__global__ __launch_bounds__(kResolveThreads, 2) void select_resolve_kernel(SelArgs a, StageWs o) {
  __shared__ ResolveSmem S;
  __shared__ int wsum[kResolveWaves];
  __shared__ int res[4][4];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool want_slots = a.sel_slot != nullptr;
  // ---- round 1: G(64 j) = the sum over chunks of cnt_ge[c][64 j] (lane =
  // chunk, wave v takes j = v + 8 m), and this chunk's page ids.  The loads
  // are issued before the length and k are known (every column of the coarse
  // table is inside the workspace; columns past the sequence's chunks are
  // masked).
  uint32_t g1[8];
  {
    const uint16_t *crow = o.coarse + (size_t)b * 64 * kSplitMaxChunks + lane;
#pragma unroll
    for (int m = 0; m < 8; ++m) g1[m] = crow[(wave + kResolveWaves * m) * kSplitMaxChunks];
  }
  int pid = 0;
  if (want_slots && t < kChunk / kPageSize)
    pid = a.page_table[(size_t)b * a.max_pages + min(w * (kChunk / kPageSize) + t, a.max_pages - 1)];
  const int P = sel_prefix(a, b);
  const int kk = sel_k(a, b, P);
  const int nch = (P + kChunk - 1) / kChunk;
  if (w >= max(nch, 1)) return;
  if (kk == 0) {  // (also P == 0)
    if (w == 0 && t == 0) a.sel_count[b] = 0;
    return;
  }
  const bool live_ln = lane < nch;
  {
#pragma unroll
    for (int m = 0; m < 8; ++m) g1[m] = live_ln ? g1[m] : 0u;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int sum = __builtin_amdgcn_readlane(wave_inclusive_scan((int)g1[m]), 63);
      if (lane == 0) S.g[wave + kResolveWaves * m] = sum;
    }
    if (t < kChunk / kPageSize) S.page[t] = pid;
    if (t < kChunk / 32) {
      S.bm[t] = 0u;
      S.tie[t] = 0u;
    }
    if (t < kSplitMaxChunks) {
      S.gt[t] = 0;
      S.eq[t] = 0;
    }
    if (t == 0) S.meta[5] = 0;
    S.h[t] = 0u;
    S.h[t + kResolveThreads] = 0u;
  }
  __syncthreads();
  // ---- round 2: G at the 65 bins base2 + l of the window the first round
  // found (lane = bin, wave v takes chunks v + 8 m; one line per load)
  const int istar = 63 - (int)__builtin_clzll(__builtin_amdgcn_ballot_w64(S.g[lane] >= kk));  // G(0) = P >= kk
  const int base2 = 64 * istar;
  uint32_t f[8], f64[8];
  {
    const uint16_t *rows = o.cnt_ge + (size_t)b * o.chunks * kCntStride;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int c = min(wave + kResolveWaves * m, nch - 1);
      const bool in = wave + kResolveWaves * m < nch;
      const uint32_t x = rows[(size_t)c * kCntStride + base2 + lane];
      const uint32_t y = rows[(size_t)c * kCntStride + min(base2 + 64, kBins1)];
      f[m] = in ? x : 0u;
      f64[m] = in ? y : 0u;
    }
    int s = 0, s64 = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      s += (int)f[m];
      s64 += (int)f64[m];
    }
    S.part[wave][lane] = s;
    if (lane == 0) S.part64[wave] = s64;
  }
  __syncthreads();  // (also: every wave has read the first round's sums)
  // every wave: G at the window's bins (lane = bin), the bin b1 holding K*
  // and the keys above it
  int jb, k1;
  {
    int g2 = 0, g64 = 0;
#pragma unroll
    for (int q = 0; q < kResolveWaves; ++q) {
      g2 += S.part[q][lane];
      g64 += S.part64[q];
    }
    jb = 63 - (int)__builtin_clzll(__builtin_amdgcn_ballot_w64(g2 >= kk));  // G(base2) >= kk
    k1 = kk - (jb < 63 ? __shfl(g2, jb + 1) : g64);  // rank of K* inside bin b1 (>= 1)
  }
  const uint32_t b1 = (uint32_t)(base2 + jb);
  // each chunk's counts at b1 and b1 + 1, from the loading lanes' registers
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int c = wave + kResolveWaves * m;
    if (c < nch) {
      if (lane == jb) S.hi[c] = (int)f[m];
      if (lane == jb + 1) S.lo[c] = (int)f[m];
      if (jb == 63 && lane == 0) S.lo[c] = (int)f64[m];
    }
  }
  __syncthreads();
  // every wave: per chunk (lane = chunk) its candidates (the entries of bin
  // b1), their offset in the sequence's candidate list, and the 64-entry read
  // items of its candidates
  const int lo_ln = live_ln ? S.lo[lane] : 0;
  const int nc_ln = live_ln ? S.hi[lane] - lo_ln : 0;
  const int cd = wave_inclusive_scan(nc_ln);
  const int off_ln = cd - nc_ln;
  const int n_cand = __builtin_amdgcn_readlane(cd, 63);
  const int np_ln = (nc_ln + kCandPiece - 1) / kCandPiece;
  const int io_ln = wave_inclusive_scan(np_ln);  // items of chunks 0 .. lane
  const int n_items = __builtin_amdgcn_readlane(io_ln, 63);
  if (wave == 0) {
    if (live_ln) S.cand_off[lane] = off_ln;
    if (lane == 63) S.cand_off[nch] = n_cand;
  }
  const bool cached = n_cand <= kResolveCache;
  const u32x2 *stg = a.ws.cand + (size_t)b * a.max_prefix;
  // ---- round 3: this chunk's entries above b1 (their positions), and every
  // candidate into the LDS cache and the histogram of its key bits [10, 20)
  // (wave v takes items v, v + 8, ..., kItemBatch of them per batch; an
  // item's chunk and offsets are wave-uniform).  The first own load and the
  // first batch of items are in flight together; more of either is rare.
  {
    const int lo_own = __builtin_amdgcn_readlane(lo_ln, w);
    const uint32_t *own_pos = reinterpret_cast<const uint32_t *>(stg + (size_t)w * kChunk) + 1;
    auto mark_own = [&](int e, uint32_t pos) {
      if (e < lo_own) {
        const int p = (int)pos - w * kChunk;
        atomicOr(&S.bm[p >> 5], 1u << (p & 31));
      }
    };
    const uint32_t up0 = own_pos[2 * min(t, max(lo_own - 1, 0))];
    const int n_it = cached ? n_items : 0;
    auto item_batch = [&](int r0) {
      u32x2 v[kItemBatch];
      int dst[kItemBatch];
#pragma unroll
      for (int q = 0; q < kItemBatch; ++q) {
        const int it = r0 + kResolveWaves * q;
        // the first chunk whose items reach past `it` (chunk 63 if none: then !ok)
        const int c = __builtin_amdgcn_readfirstlane(
            (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(io_ln > it) | (1ull << 63)));
        const int i = kCandPiece * (it - __builtin_amdgcn_readlane(io_ln - np_ln, c)) + lane;
        const bool ok = it < n_it && i < __builtin_amdgcn_readlane(nc_ln, c);
        dst[q] = ok ? __builtin_amdgcn_readlane(off_ln, c) + i : -1;
        v[q] = stg[ok ? (size_t)c * kChunk + __builtin_amdgcn_readlane(lo_ln, c) + i : 0];
      }
#pragma unroll
      for (int q = 0; q < kItemBatch; ++q) {
        if (dst[q] >= 0) {
          S.cache[dst[q]] = v[q];
          atomicAdd(&S.h[(v[q][0] >> 10) & 1023u], 1u);  // the histogram of key bits [10, 20)
        }
      }
    };
    if (wave < n_it) item_batch(wave);
    mark_own(t, up0);
    for (int r0 = wave + kResolveWaves * kItemBatch; r0 < n_it; r0 += kResolveWaves * kItemBatch) item_batch(r0);
    for (int e = t + kResolveThreads; e < lo_own; e += kResolveThreads) mark_own(e, own_pos[2 * e]);
  }
  __syncthreads();
  // candidate i (0 <= i < n_cand) of the sequence
  auto cand = [&](int i) -> u32x2 {
    if (cached) return S.cache[i];
    int c = 0;
    while (S.cand_off[c + 1] <= i) ++c;
    return stg[(size_t)c * kChunk + S.lo[c] + (i - S.cand_off[c])];
  };
  // ---- K* from the candidates: bits [10, 20) (histogram built as the cached
  // candidates arrived), then [0, 10)
  if (!cached) {
    for (int i = t; i < n_cand; i += kResolveThreads) atomicAdd(&S.h[(cand(i)[0] >> 10) & 1023u], 1u);
    __syncthreads();
  }
  uint32_t hb[2] = {S.h[kBins23 - 1 - 2 * t], S.h[kBins23 - 2 - 2 * t]};
  int above2, n_b2;
  const uint32_t b2 = (uint32_t)find_bin_n<kResolveWaves, 2>(hb, kBins23, k1, wsum, res[0], above2, n_b2);
  const int k2 = k1 - above2;  // rank of K* inside bin b2 (>= 1)
  const uint32_t pre22 = (b1 << 10) | b2;
  int ties = 0;                 // keys equal to K* to keep, lowest positions first (wave 0)
  int x_gt = 0, x_eq = 0;       // wave 0: chunk `lane`'s keys above / equal to K* from the list
  uint32_t x_bm = 0u, x_tie = 0u;  // wave 0: bits of this chunk's bitmap word `lane` from the list
  if (n_b2 <= kWave) {
    // Few keys share K*'s top 22 bits: one pass over the candidates counts
    // the keys above that bin per chunk (and marks this chunk's) and lists
    // the bin's keys; wave 0 ranks the list.
    for (int i = t; i < n_cand; i += kResolveThreads) {
      const u32x2 e = cand(i);
      const uint32_t h22 = e[0] >> 10;
      if (h22 > pre22) {
        const int c = (int)(e[1] >> 11);
        atomicAdd(&S.gt[c], 1);
        if (c == w) atomicOr(&S.bm[(e[1] & (kChunk - 1)) >> 5], 1u << (e[1] & 31));
      } else if (h22 == pre22) {
        S.list[atomicAdd(&S.meta[5], 1)] = e;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const u32x2 mine = S.list[min(lane, n_b2 - 1)];
      int gt_j = 0, ge_j = 0;  // list keys above / at least this lane's
      for (int l = 0; l < n_b2; ++l) {
        const uint32_t kl = S.list[l][0];
        gt_j += kl > mine[0];
        ge_j += kl >= mine[0];
      }
      // K* is the key of every lane with gt_j < k2 <= ge_j
      const int src = __ffsll((unsigned long long)__builtin_amdgcn_ballot_w64(lane < n_b2 && gt_j < k2 && k2 <= ge_j)) - 1;
      const uint32_t kstar = (uint32_t)__shfl((int)mine[0], src);
      ties = k2 - __shfl(gt_j, src);
      for (int l = 0; l < n_b2; ++l) {
        const u32x2 e = S.list[l];
        const int c = (int)(e[1] >> 11);
        const bool gt = e[0] > kstar, eq = e[0] == kstar;
        x_gt += (gt && c == lane);
        x_eq += (eq && c == lane);
        if (c == w && (int)((e[1] & (kChunk - 1)) >> 5) == lane) {
          if (gt) x_bm |= 1u << (e[1] & 31);
          if (eq) x_tie |= 1u << (e[1] & 31);
        }
      }
    }
  } else {
    S.h[kBins23 - 1 - 2 * t] = 0u;  // each thread clears the bins it read
    S.h[kBins23 - 2 - 2 * t] = 0u;
    __syncthreads();
    for (int i = t; i < n_cand; i += kResolveThreads) {
      const uint32_t key = cand(i)[0];
      if ((key >> 10) == pre22) atomicAdd(&S.h[key & 1023u], 1u);
    }
    __syncthreads();
    hb[0] = S.h[kBins23 - 1 - 2 * t];
    hb[1] = S.h[kBins23 - 2 - 2 * t];
    int above3, n_eq;
    const uint32_t b3 = (uint32_t)find_bin_n<kResolveWaves, 2>(hb, kBins23, k2, wsum, res[1], above3, n_eq);
    const uint32_t kstar = (pre22 << 10) | b3;
    ties = k2 - above3;
    // per chunk: candidates above and equal to K* (a candidate's chunk is its
    // position / 2048); this chunk's own go to its bitmaps
    for (int i = t; i < n_cand; i += kResolveThreads) {
      const u32x2 e = cand(i);
      const int c = (int)(e[1] >> 11);
      if (e[0] > kstar) {
        atomicAdd(&S.gt[c], 1);
        if (c == w) atomicOr(&S.bm[(e[1] & (kChunk - 1)) >> 5], 1u << (e[1] & 31));
      } else if (e[0] == kstar) {
        atomicAdd(&S.eq[c], 1);
        if (c == w) atomicOr(&S.tie[(e[1] & (kChunk - 1)) >> 5], 1u << (e[1] & 31));
      }
    }
    __syncthreads();
  }
  // ---- wave 0 (the others are done): the chunk's output offset and its
  // share of the ties, its positions in order (lane = bitmap word of 32
  // positions), then their writes
  if (wave != 0) return;
  const int eq = live_ln ? S.eq[lane] + x_eq : 0;
  const int eq_before = wave_inclusive_scan(eq) - eq;
  const int take = min(eq, max(0, ties - eq_before));  // ties taken in this chunk
  const int sel = live_ln ? lo_ln + S.gt[lane] + x_gt + take : 0;
  const int off = wave_inclusive_scan(sel) - sel;
  const int my_off = __shfl(off, w), my_take = __shfl(take, w);
  // this chunk's ties: the first my_take tie bits in position order
  uint32_t tw = S.tie[lane] | x_tie;
  const int tc = __popc(tw);
  int rank = wave_inclusive_scan(tc) - tc;
  uint32_t x = tw;
  while (x) {
    const uint32_t bit = x & (~x + 1u);
    if (rank >= my_take) tw &= ~bit;
    ++rank;
    x &= x - 1u;
  }
  uint32_t word = S.bm[lane] | x_bm | tw;
  const int cnt = __popc(word);
  int idx = wave_inclusive_scan(cnt) - cnt;
  const int n_own = __builtin_amdgcn_readlane(idx + cnt, 63);  // this chunk's selected count
  while (word) {
    const int bit = __ffs(word) - 1;
    word &= word - 1u;
    S.out[idx++] = w * kChunk + 32 * lane + bit;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int32_t *pos_row = a.sel_pos + (size_t)b * a.max_k;
  int32_t *slot_row = want_slots ? a.sel_slot + (size_t)b * a.max_k : nullptr;
  for (int j = lane; j < n_own; j += kWave) {
    const int i = my_off + j;
    if (i < a.max_k) {
      const int pos = S.out[j];
      pos_row[i] = pos;
      if (want_slots) slot_row[i] = S.page[(pos & (kChunk - 1)) >> 4] * kPageSize + (pos & (kPageSize - 1));
    }
  }
  if (w == 0 && lane == 0) a.sel_count[b] = kk;
}

}  // namespace vg
