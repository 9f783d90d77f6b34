// vegas_attn.hip -- host side of the vegas_attn C-ABI: argument validation,
// workspace layout, launch planning and kernel launches.  See
// include/vegas_attn.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "vegas_attn.h"
#include "attn_common.h"
#include "launch.h"
#include "select.h"
#include "select_split.h"
#include "kv_append.h"
#include "window_select.h"

namespace {

using namespace vg;

constexpr size_t kAlign = 256;
constexpr int kCUs = 256;  // MI355X compute units

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

__global__ void zero_kernel(u32x4 *p, size_t n16, uint8_t *tail, size_t ntail) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p[j] = u32x4{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0;
}

bool valid_shape(const vg_shape *s) {
  if (!s) return false;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1) return false;
  if (s->num_q_heads % s->num_kv_heads) return false;
  if (s->head_dim < 1 || s->page_size < 1 || s->max_pages_per_seq < 1) return false;
  if (s->dtype != VG_DTYPE_F32 && s->dtype != VG_DTYPE_BF16) return false;
  if (s->kernel < VG_KERNEL_AUTO || s->kernel > VG_KERNEL_MFMA) return false;
  if (!std::isfinite(s->softmax_scale)) return false;
  return true;
}

vg_status supported_shape(const vg_shape *s) {
  if (s->head_dim != 64 && s->head_dim != 128) return VG_ERR_UNSUPPORTED;
  if (s->page_size != kPageSize) return VG_ERR_UNSUPPORTED;
  if (s->dtype == VG_DTYPE_F32 && s->kernel == VG_KERNEL_MFMA) return VG_ERR_UNSUPPORTED;
  return VG_OK;
}

bool use_mfma(const vg_shape *s) {
  return s->dtype == VG_DTYPE_BF16 && s->kernel != VG_KERNEL_VALU;
}

// Launch plan and workspace layout of one attention call.  Verify lists are
// long and may be ragged: the workgroups share their tiles evenly (stream-K).
// Sparse draft lists are short: fixed splits.
struct AttnPlan {
  int rows, nt, mr, tile, workgroups, split_tokens, splits;
  long long share_entries;  // verify: the most entries one workgroup's share can hold
  bool mfma, ok;  // ok: batch and tile counts within the kernels' limits
  size_t off_part_o, off_part_ml, bytes;
};

AttnPlan plan_attention(const vg_shape *s, int nrows, long long max_len, bool sparse) {
  AttnPlan p{};
  const int G = s->num_q_heads / s->num_kv_heads;
  p.rows = nrows * G;
  p.nt = (p.rows + 15) / 16;
  p.mr = p.rows <= 16 ? 16 : (p.rows <= 32 ? 32 : 64);
  p.mfma = use_mfma(s);
  p.tile = p.mfma ? 32 : kWave;
  const long long bg = (long long)s->batch * s->num_kv_heads;
  const long long L = max_len > 0 ? max_len : 1;
  long long n_part;
  p.ok = s->batch <= kMaxBatch && bg * ((L + p.tile - 1) / p.tile) < (1LL << 31);
  if (sparse) {
    // Sparse draft lists are short and the call is latency-bound: fixed splits
    // of 4 tiles (one per wave) while all workgroups fit the kernel's
    // residency, else of 8 tiles.  Where that leaves some CUs with two
    // workgroups and others with one, the splits shrink to the smallest size
    // that still keeps every workgroup resident: the busiest CU then has
    // fewer tiles (C3: splits of 3 tiles on 440 workgroups instead of 4 on
    // 336, 11.4 against 11.8 us per draft step).  Fixed splits need no length
    // lookup before the first load; workgroups past a list's end exit after
    // writing an empty partial, and the hardware dispatcher balances ragged
    // batches.
    const long long res = (long long)(p.mfma ? attn_occupancy(s->head_dim, p.nt, VG_SPARSE_PF, true) : 1) * kCUs;
    const long long tiles = (L + p.tile - 1) / p.tile;  // of the longest list
    long long split = bg * ((tiles + kWaves - 1) / kWaves) <= res ? kWaves : 2 * kWaves;  // in tiles
    const long long wgs = bg * ((tiles + split - 1) / split);
    if (wgs > kCUs && wgs <= res) {
      const long long per_list = std::max(1LL, res / bg);
      split = std::min(split, (tiles + per_list - 1) / per_list);
    }
    p.split_tokens = (int)(split * p.tile);
    p.splits = (int)((L + p.split_tokens - 1) / p.split_tokens);
    p.workgroups = (int)(bg * p.splits);
    n_part = p.workgroups;
  } else {
    // one wave of resident workgroups (1 per CU), at least one tile per wave
    const long long tiles = bg * ((L + p.tile - 1) / p.tile);
    const int occ = !p.mfma ? 1 : attn_occupancy(s->head_dim, p.nt, verify_pf(s->head_dim, p.nt), false);
    const int resident = occ * kCUs;
    p.workgroups = (int)std::min<long long>((tiles + kWaves - 1) / kWaves, resident);
    p.share_entries = (tiles + p.workgroups - 1) / p.workgroups * p.tile;
    p.split_tokens = 0;
    p.splits = 0;
    n_part = p.workgroups + bg;
  }
  p.off_part_o = 0;
  p.off_part_ml = align_up((size_t)n_part * p.rows * s->head_dim * sizeof(float));
  p.bytes = p.off_part_ml + align_up((size_t)n_part * p.rows * 2 * sizeof(float));
  return p;
}

float effective_scale(const vg_shape *s) {
  return s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / std::sqrt((float)s->head_dim);
}


template <int D>
void launch_combine(int rpb, const AttnArgs &a, dim3 grid, hipStream_t st) {
  switch (rpb) {
    case 1: hipLaunchKernelGGL((combine_kernel<D, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((combine_kernel<D, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((combine_kernel<D, 4>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((combine_kernel<D, 8>), grid, dim3(kThreads), 0, st, a); break;
  }
}

// Rows per combine block: as many as leave each row enough partial groups
// to load its (at most) np partials in one batch of 8 per thread.
int combine_rows_per_block(const vg_shape *s, const AttnPlan &p) {
  const int cols = s->head_dim / 4;
  const long long bg = (long long)s->batch * s->num_kv_heads;
  const long long np = p.split_tokens > 0 ? p.splits : (p.workgroups + bg - 1) / bg + 1;
  int rpb = 1;
  while (rpb < 8 && (kThreads / (2 * rpb)) / cols * 8 >= np && kThreads / (2 * rpb) >= cols) rpb *= 2;
  return rpb;
}

// Attention kernel over the shared key lists, then (with_combine) combine
// blocks of one or more rows per (KV head, sequence).
vg_status launch_attention(const vg_shape *s, const AttnPlan &p, AttnArgs &a, char *ws,
                           hipStream_t st, bool with_combine = true) {
  a.part_o = reinterpret_cast<float *>(ws + p.off_part_o);
  a.part_ml = reinterpret_cast<float *>(ws + p.off_part_ml);
  a.batch = s->batch;
  a.workgroups = p.workgroups;
  a.tile = p.tile;
  a.split_tokens = p.split_tokens;
  a.splits = p.splits;
  a.rows = p.rows;
  const dim3 grid(p.workgroups);
  if (p.mfma) {
    if (s->head_dim == 128) {
      if (a.sparse) launch_mfma128_sparse(p.nt, a, grid, st);
      else launch_mfma128_verify(p.nt, a, grid, st, p.share_entries);
    } else {
      if (a.sparse) launch_mfma64_sparse(p.nt, a, grid, st);
      else launch_mfma64_verify(p.nt, a, grid, st);
    }
  } else {
    const bool bf16 = s->dtype == VG_DTYPE_BF16;
    if (s->head_dim == 128) {
      if (bf16) launch_valu_bf16128(p.mr, a, grid, st);
      else launch_valu_f32128(p.mr, a, grid, st);
    } else {
      if (bf16) launch_valu_bf1664(p.mr, a, grid, st);
      else launch_valu_f3264(p.mr, a, grid, st);
    }
  }
  if (!with_combine) return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
  const int rpb = combine_rows_per_block(s, p);
  const dim3 cgrid((p.rows + rpb - 1) / rpb, s->num_kv_heads, s->batch);
  if (s->head_dim == 128) launch_combine<128>(rpb, a, cgrid, st);
  else launch_combine<64>(rpb, a, cgrid, st);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

// ---------------------------------------------------------------- topk workspace
struct SelPlan {
  size_t off_hist1, off_hist2, off_state, off_above, off_ncand, off_cand, off_cntge, off_coarse, bytes;
  int chunks;  // chunks of kChunk positions per sequence
};

// Two-launch selection (select_split.h): prefixes up to kSplitMaxPrefix with
// even rows (8-byte score loads), and slots through 16-token pages.
bool split_ok(int batch, int max_prefix, bool slots, int page_size) {
  return max_prefix <= kSplitMaxPrefix && max_prefix % 2 == 0 && batch <= 65535 &&
         (!slots || page_size == kPageSize);
}

SelPlan plan_select(int batch, int max_prefix) {
  SelPlan p{};
  p.chunks = ceil_div(max_prefix > 0 ? max_prefix : 1, kChunk);
  p.off_hist1 = 0;
  p.off_hist2 = align_up((size_t)batch * kBins1 * sizeof(uint32_t));
  p.off_state = p.off_hist2 + align_up((size_t)batch * kBins23 * sizeof(uint32_t));
  p.off_above = p.off_state + align_up((size_t)batch * 4 * sizeof(int32_t));
  p.off_ncand = p.off_above + align_up((size_t)batch * kMaxChunks * sizeof(int32_t));
  p.off_cand = p.off_ncand + align_up((size_t)batch * kMaxChunks * sizeof(int32_t));
  p.off_cntge = p.off_cand + align_up((size_t)batch * (size_t)(max_prefix > 0 ? max_prefix : 1) * 8);
  const bool split = max_prefix <= kSplitMaxPrefix;
  p.off_coarse = p.off_cntge + (split ? align_up((size_t)batch * p.chunks * kCntStride * sizeof(uint16_t)) : 0);
  p.bytes = p.off_coarse + (split ? align_up((size_t)batch * 64 * kSplitMaxChunks * sizeof(uint16_t)) : 0);
  return p;
}

StageWs stage_ws(const SelPlan &p, void *ws) {
  char *c = static_cast<char *>(ws);
  StageWs o;
  o.cnt_ge = reinterpret_cast<uint16_t *>(c + p.off_cntge);
  o.coarse = reinterpret_cast<uint16_t *>(c + p.off_coarse);
  o.chunks = p.chunks;
  return o;
}

SelWs sel_ws(const SelPlan &p, void *ws) {
  char *c = static_cast<char *>(ws);
  SelWs w;
  w.hist1 = reinterpret_cast<uint32_t *>(c + p.off_hist1);
  w.hist2 = reinterpret_cast<uint32_t *>(c + p.off_hist2);
  w.state = reinterpret_cast<int32_t *>(c + p.off_state);
  w.above = reinterpret_cast<int32_t *>(c + p.off_above);
  w.ncand = reinterpret_cast<int32_t *>(c + p.off_ncand);
  w.cand = reinterpret_cast<u32x2 *>(c + p.off_cand);
  return w;
}

constexpr int kMaxSelectPrefix = kMaxChunks * kChunk;

// Validation and launch arguments of a verify call (vg_verify_attention and
// the calls built on it).
vg_status verify_prepare(const vg_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *page_table, const int32_t *prefix_len, int32_t max_prefix,
                         int32_t gamma, float *out, float *logits, float *group_scores, void *workspace,
                         size_t workspace_bytes, bool export_all, AttnPlan &p, AttnArgs &a) {
  if (!valid_shape(shape) || max_prefix < 0 || gamma < 0 || gamma > 15) return VG_ERR_INVALID_ARG;
  const void *req[] = {q, k_cache, v_cache, page_table, prefix_len, out};
  for (const void *ptr : req)
    if (!ptr || !aligned16(ptr)) return VG_ERR_INVALID_ARG;
  if ((logits && !aligned16(logits)) || (group_scores && !aligned16(group_scores)))
    return VG_ERR_INVALID_ARG;
  const vg_status sup = supported_shape(shape);
  if (sup != VG_OK) return sup;
  const int R = gamma + 1;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (R * G > kMaxRows) return VG_ERR_UNSUPPORTED;
  if (ceil_div((long long)max_prefix + R, shape->page_size) > shape->max_pages_per_seq)
    return VG_ERR_INVALID_ARG;
  p = plan_attention(shape, R, (long long)max_prefix + R, false);
  if (!p.ok) return VG_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) || workspace_bytes < p.bytes) return VG_ERR_WORKSPACE;
  a = AttnArgs{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.prefix_len = prefix_len;
  a.out = out;
  a.logits = logits;
  a.group = group_scores;
  a.max_pages = shape->max_pages_per_seq;
  a.max_prefix = max_prefix;
  a.nrows = R;
  a.gamma = gamma;
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.group_size = G;
  a.scale = effective_scale(shape);
  a.scale_log2 = a.scale * kLog2e;
  a.sparse = 0;
  a.export_all = export_all ? 1 : 0;
  return VG_OK;
}

vg_status verify_impl(const vg_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *page_table, const int32_t *prefix_len, int32_t max_prefix,
                      int32_t gamma, float *out, float *logits, float *group_scores, void *workspace,
                      size_t workspace_bytes, void *stream, bool export_all) {
  AttnPlan p;
  AttnArgs a;
  const vg_status st = verify_prepare(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma, out,
                                      logits, group_scores, workspace, workspace_bytes, export_all, p, a);
  if (st != VG_OK) return st;
  return launch_attention(shape, p, a, static_cast<char *>(workspace), static_cast<hipStream_t>(stream));
}

// The verify call's second kernel with the selection's first step beside it:
// blocks [0, nstage) stage one chunk of the group export each (stage_block),
// the others are the verify combine's blocks (grid (ncomb_x, Hkv, B),
// flattened).  The export is complete when this kernel starts: the attention
// kernel before it wrote it.
template <int D, int RPB>
__global__ __launch_bounds__(kThreads) void combine_stage_kernel(AttnArgs a, SelArgs s, StageWs o, int ncomb_x,
                                                                int nstage_x) {
  const int id = blockIdx.x, nstage = nstage_x * s.batch;
  if (id < nstage) {
    stage_block<true, kThreads>(s, o, id / nstage_x, id % nstage_x);
    return;
  }
  const int c = id - nstage, Hkv = a.num_kv_heads;
  combine_block<D, RPB>(a, c % ncomb_x, (c / ncomb_x) % Hkv, c / (ncomb_x * Hkv));
}

// rpb: rows per combine block (combine_rows_per_block).
template <int D>
void launch_combine_stage(int rpb, const AttnArgs &a, const SelArgs &s, const StageWs &o, int nstage_x,
                          hipStream_t st) {
  const int ncomb_x = (a.rows + rpb - 1) / rpb;
  const dim3 grid(nstage_x * s.batch + ncomb_x * a.num_kv_heads * a.batch);
  switch (rpb) {
    case 1: hipLaunchKernelGGL((combine_stage_kernel<D, 1>), grid, dim3(kThreads), 0, st, a, s, o, ncomb_x, nstage_x); break;
    case 2: hipLaunchKernelGGL((combine_stage_kernel<D, 2>), grid, dim3(kThreads), 0, st, a, s, o, ncomb_x, nstage_x); break;
    case 4: hipLaunchKernelGGL((combine_stage_kernel<D, 4>), grid, dim3(kThreads), 0, st, a, s, o, ncomb_x, nstage_x); break;
    default: hipLaunchKernelGGL((combine_stage_kernel<D, 8>), grid, dim3(kThreads), 0, st, a, s, o, ncomb_x, nstage_x); break;
  }
}

// ---------------------------------------------------------------- scratch
// Workspace of vg_sparse_draft_attention_noalloc: a file-scope device array,
// one copy per GPU the library runs on, held until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): it looks up the device address once per device,
// with that device current, and uses that pointer.
constexpr size_t kScratchBytes = VG_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

vg_status scratch_on_current_device(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VG_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return VG_ERR_HIP;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return VG_OK;
}

vg_status sparse_impl(const vg_shape *shape, const void *q, int32_t n_q,
                      const void *k_cache, const void *v_cache,
                      const int32_t *sel_slot, const int32_t *sel_count,
                      int32_t max_k, const int32_t *page_table,
                      const int32_t *tail_start, const int32_t *tail_len,
                      int32_t max_tail, float *out, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!valid_shape(shape) || n_q < 1 || max_k < 0 || max_tail < n_q) return VG_ERR_INVALID_ARG;
  const void *req[] = {q, k_cache, v_cache, sel_count, page_table, tail_start, tail_len, out};
  for (const void *p : req)
    if (!p || !aligned16(p)) return VG_ERR_INVALID_ARG;
  if (max_k > 0 && (!sel_slot || !aligned16(sel_slot))) return VG_ERR_INVALID_ARG;
  const vg_status sup = supported_shape(shape);
  if (sup != VG_OK) return sup;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (n_q * G > kMaxRows) return VG_ERR_UNSUPPORTED;
  const AttnPlan p = plan_attention(shape, n_q, (long long)max_k + max_tail, true);
  if (!p.ok) return VG_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) || workspace_bytes < p.bytes) return VG_ERR_WORKSPACE;
  AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.sel_slot = sel_slot;
  a.sel_count = sel_count;
  a.tail_start = tail_start;
  a.tail_len = tail_len;
  a.out = out;
  a.max_pages = shape->max_pages_per_seq;
  a.max_k = max_k;
  a.max_tail = max_tail;
  a.nrows = n_q;
  a.gamma = 0;
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.group_size = G;
  a.scale = effective_scale(shape);
  a.scale_log2 = a.scale * kLog2e;
  a.sparse = 1;
  return launch_attention(shape, p, a, static_cast<char *>(workspace),
                          static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

const char *vg_status_string(vg_status status) {
  switch (status) {
    case VG_OK: return "VG_OK";
    case VG_ERR_INVALID_ARG: return "VG_ERR_INVALID_ARG";
    case VG_ERR_UNSUPPORTED: return "VG_ERR_UNSUPPORTED";
    case VG_ERR_WORKSPACE: return "VG_ERR_WORKSPACE";
    case VG_ERR_HIP: return "VG_ERR_HIP";
    default: return "VG_ERR_UNKNOWN";
  }
}

const char *vg_version(void) { return "vegas_attn 0.1 (gfx950)"; }

vg_status vg_workspace_zero(void *workspace, size_t bytes, void *stream) {
  if (bytes == 0) return VG_OK;
  if (!workspace || !aligned16(workspace)) return VG_ERR_INVALID_ARG;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  uint8_t *tail = static_cast<uint8_t *>(workspace) + n16 * 16;
  const int blocks = (int)std::min<size_t>(4096, (n16 + 255) / 256 + 1);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4 *>(workspace), n16, tail, ntail);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_verify_workspace_size(const vg_shape *shape, int32_t max_prefix, int32_t gamma,
                                   size_t *bytes) {
  if (!bytes || !valid_shape(shape) || max_prefix < 0 || gamma < 0 || gamma > 15)
    return VG_ERR_INVALID_ARG;
  const vg_status sup = supported_shape(shape);
  if (sup != VG_OK) return sup;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if ((gamma + 1) * G > kMaxRows) return VG_ERR_UNSUPPORTED;
  const AttnPlan p = plan_attention(shape, gamma + 1, (long long)max_prefix + gamma + 1, false);
  if (!p.ok) return VG_ERR_UNSUPPORTED;
  *bytes = p.bytes;
  return VG_OK;
}

vg_status vg_verify_attention(const vg_shape *shape, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *page_table,
                              const int32_t *prefix_len, int32_t max_prefix, int32_t gamma,
                              float *out, float *logits, float *group_scores, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return verify_impl(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma, out, logits,
                     group_scores, workspace, workspace_bytes, stream, false);
}

vg_status vg_verify_attention_all_rows(const vg_shape *shape, const void *q, const void *k_cache,
                                       const void *v_cache, const int32_t *page_table,
                                       const int32_t *prefix_len, int32_t max_prefix, int32_t gamma,
                                       float *out, float *logits, float *group_scores,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  return verify_impl(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma, out, logits,
                     group_scores, workspace, workspace_bytes, stream, true);
}

vg_status vg_aggregate_scores(int32_t batch, const float *src, int32_t src_rows, int32_t src_heads,
                              const int32_t *prefix_len, int32_t max_prefix, float *scores,
                              void *select_ws, size_t select_ws_bytes, void *stream) {
  if (batch < 1 || src_rows < 1 || src_heads < 1 || max_prefix < 0) return VG_ERR_INVALID_ARG;
  if (!src || !prefix_len || !scores || !aligned16(src) || !aligned16(prefix_len) ||
      !aligned16(scores))
    return VG_ERR_INVALID_ARG;
  if (max_prefix > kMaxSelectPrefix) return VG_ERR_UNSUPPORTED;
  SelArgs a{};
  a.batch = batch;
  a.max_prefix = max_prefix;
  a.prefix_len = prefix_len;
  a.scores_out = scores;
  a.src = src;
  a.src_rows = src_rows;
  a.src_heads = src_heads;
  if (max_prefix == 0) return VG_OK;
  const dim3 grid(ceil_div(max_prefix, kP1Block), batch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (select_ws) {
    const SelPlan p = plan_select(batch, max_prefix);
    if (!aligned16(select_ws) || select_ws_bytes < p.bytes) return VG_ERR_WORKSPACE;
    a.ws = sel_ws(p, select_ws);
    hipLaunchKernelGGL((select_pass1_kernel<true, true>), grid, dim3(kP1Threads), 0, st, a);
  } else {
    hipLaunchKernelGGL((select_pass1_kernel<true, false>), grid, dim3(kP1Threads), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_topk_workspace_size(int32_t batch, int32_t max_prefix, size_t *bytes) {
  if (!bytes || batch < 1 || max_prefix < 0) return VG_ERR_INVALID_ARG;
  if (max_prefix > kMaxSelectPrefix) return VG_ERR_UNSUPPORTED;
  *bytes = plan_select(batch, max_prefix).bytes;
  return VG_OK;
}

vg_status vg_topk_select(int32_t batch, const float *scores, int32_t max_prefix,
                         const int32_t *prefix_len, const int32_t *k, int32_t max_k,
                         const int32_t *page_table, int32_t page_size, int32_t max_pages_per_seq,
                         int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count, int32_t flags,
                         void *workspace, size_t workspace_bytes, void *stream) {
  if (batch < 1 || max_prefix < 0 || max_k < 0) return VG_ERR_INVALID_ARG;
  if (flags != 0 && flags != VG_TOPK_PREPASS_DONE) return VG_ERR_INVALID_ARG;
  const void *req[] = {scores, prefix_len, k, sel_pos, sel_count};
  for (const void *p : req)
    if (!p || !aligned16(p)) return VG_ERR_INVALID_ARG;
  if (sel_slot && (!aligned16(sel_slot) || !page_table || !aligned16(page_table) ||
                   page_size < 1 || max_pages_per_seq < 1 ||
                   ceil_div(max_prefix, page_size) > max_pages_per_seq))
    return VG_ERR_INVALID_ARG;
  if (max_prefix > kMaxSelectPrefix) return VG_ERR_UNSUPPORTED;
  const SelPlan p = plan_select(batch, max_prefix);
  if (!workspace || !aligned16(workspace) || workspace_bytes < p.bytes) return VG_ERR_WORKSPACE;
  SelArgs a{};
  a.batch = batch;
  a.max_prefix = max_prefix;
  a.max_k = max_k;
  a.prefix_len = prefix_len;
  a.k = k;
  a.scores = scores;
  a.page_table = page_table;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  a.sel_pos = sel_pos;
  a.sel_slot = sel_slot;
  a.sel_count = sel_count;
  a.ws = sel_ws(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(ceil_div(max_prefix > 0 ? max_prefix : 1, kChunk), batch);
  if (!(flags & VG_TOPK_PREPASS_DONE) && split_ok(batch, max_prefix, sel_slot != nullptr, page_size)) {
    const StageWs o = stage_ws(p, workspace);
    hipLaunchKernelGGL((select_stage_kernel<false>), grid, dim3(kStageThreads), 0, st, a, o);
    hipLaunchKernelGGL(select_resolve_kernel, grid, dim3(kResolveThreads), 0, st, a, o);
    return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
  }
  const dim3 grid1(ceil_div(max_prefix > 0 ? max_prefix : 1, kP1Block), batch);
  if (!(flags & VG_TOPK_PREPASS_DONE))
    hipLaunchKernelGGL((select_pass1_kernel<false, true>), grid1, dim3(kP1Threads), 0, st, a);
  hipLaunchKernelGGL(select_pass2_kernel, grid, dim3(kSelThreads), 0, st, a);
  hipLaunchKernelGGL(select_pass3_kernel, grid, dim3(kSelThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_aggregate_topk_select(int32_t batch, const float *src, int32_t src_rows, int32_t src_heads,
                                   const int32_t *prefix_len, int32_t max_prefix, float *scores,
                                   const int32_t *k, int32_t max_k, const int32_t *page_table,
                                   int32_t page_size, int32_t max_pages_per_seq, int32_t *sel_pos,
                                   int32_t *sel_slot, int32_t *sel_count, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  if (batch < 1 || src_rows < 1 || src_heads < 1 || max_prefix < 0 || max_k < 0) return VG_ERR_INVALID_ARG;
  const void *req[] = {src, prefix_len, scores, k, sel_pos, sel_count};
  for (const void *ptr : req)
    if (!ptr || !aligned16(ptr)) return VG_ERR_INVALID_ARG;
  if (sel_slot && (!aligned16(sel_slot) || !page_table || !aligned16(page_table) || page_size < 1 ||
                   max_pages_per_seq < 1 || ceil_div(max_prefix, page_size) > max_pages_per_seq))
    return VG_ERR_INVALID_ARG;
  if (max_prefix > kMaxSelectPrefix) return VG_ERR_UNSUPPORTED;
  const SelPlan p = plan_select(batch, max_prefix);
  if (!workspace || !aligned16(workspace) || workspace_bytes < p.bytes) return VG_ERR_WORKSPACE;
  SelArgs a{};
  a.batch = batch;
  a.max_prefix = max_prefix;
  a.max_k = max_k;
  a.prefix_len = prefix_len;
  a.k = k;
  a.scores = scores;
  a.scores_out = scores;
  a.src = src;
  a.src_rows = src_rows;
  a.src_heads = src_heads;
  a.page_table = page_table;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  a.sel_pos = sel_pos;
  a.sel_slot = sel_slot;
  a.sel_count = sel_count;
  a.ws = sel_ws(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(ceil_div(max_prefix > 0 ? max_prefix : 1, kChunk), batch);
  if (split_ok(batch, max_prefix, sel_slot != nullptr, page_size)) {
    const StageWs o = stage_ws(p, workspace);
    hipLaunchKernelGGL((select_stage_kernel<true>), grid, dim3(kStageThreads), 0, st, a, o);
    hipLaunchKernelGGL(select_resolve_kernel, grid, dim3(kResolveThreads), 0, st, a, o);
  } else {
    const dim3 grid1(ceil_div(max_prefix > 0 ? max_prefix : 1, kP1Block), batch);
    hipLaunchKernelGGL((select_pass1_kernel<true, true>), grid1, dim3(kP1Threads), 0, st, a);
    hipLaunchKernelGGL(select_pass2_kernel, grid, dim3(kSelThreads), 0, st, a);
    hipLaunchKernelGGL(select_pass3_kernel, grid, dim3(kSelThreads), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_verify_select(const vg_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *page_table, const int32_t *prefix_len, int32_t max_prefix, int32_t gamma,
                           float *out, float *group_scores, float *scores, const int32_t *k, int32_t max_k,
                           int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count, void *verify_ws,
                           size_t verify_ws_bytes, void *select_ws, size_t select_ws_bytes, void *stream) {
  if (!group_scores) return VG_ERR_INVALID_ARG;
  AttnPlan p;
  AttnArgs a;
  const vg_status vst = verify_prepare(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma, out,
                                       nullptr, group_scores, verify_ws, verify_ws_bytes, false, p, a);
  if (vst != VG_OK) return vst;
  if (max_k < 0) return VG_ERR_INVALID_ARG;
  const void *req[] = {scores, k, sel_pos, sel_count};
  for (const void *ptr : req)
    if (!ptr || !aligned16(ptr)) return VG_ERR_INVALID_ARG;
  if (sel_slot && !aligned16(sel_slot)) return VG_ERR_INVALID_ARG;
  if (max_prefix > kMaxSelectPrefix) return VG_ERR_UNSUPPORTED;
  const int B = shape->batch, Hkv = shape->num_kv_heads;
  const SelPlan sp = plan_select(B, max_prefix);
  if (!select_ws || !aligned16(select_ws) || select_ws_bytes < sp.bytes) return VG_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!split_ok(B, max_prefix, sel_slot != nullptr, shape->page_size)) {
    // the same work as the separate calls
    const vg_status st = launch_attention(shape, p, a, static_cast<char *>(verify_ws), hs);
    if (st != VG_OK) return st;
    return vg_aggregate_topk_select(B, group_scores, 1, Hkv, prefix_len, max_prefix, scores, k, max_k, page_table,
                                    shape->page_size, shape->max_pages_per_seq, sel_pos, sel_slot, sel_count,
                                    select_ws, select_ws_bytes, stream);
  }
  SelArgs sa{};
  sa.batch = B;
  sa.max_prefix = max_prefix;
  sa.max_k = max_k;
  sa.prefix_len = prefix_len;
  sa.k = k;
  sa.scores = scores;
  sa.scores_out = scores;
  sa.src = group_scores;
  sa.src_rows = 1;
  sa.src_heads = Hkv;
  sa.page_table = page_table;
  sa.page_size = shape->page_size;
  sa.max_pages = shape->max_pages_per_seq;
  sa.sel_pos = sel_pos;
  sa.sel_slot = sel_slot;
  sa.sel_count = sel_count;
  sa.ws = sel_ws(sp, select_ws);
  const StageWs o = stage_ws(sp, select_ws);
  // attention kernel; then combine and the selection's staging in one launch;
  // then the selection's resolve
  const vg_status st = launch_attention(shape, p, a, static_cast<char *>(verify_ws), hs, false);
  if (st != VG_OK) return st;
  const int rpb = combine_rows_per_block(shape, p);
  if (shape->head_dim == 128) launch_combine_stage<128>(rpb, a, sa, o, sp.chunks, hs);
  else launch_combine_stage<64>(rpb, a, sa, o, sp.chunks, hs);
  hipLaunchKernelGGL(select_resolve_kernel, dim3(sp.chunks, B), dim3(kResolveThreads), 0, hs, sa, o);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_sparse_draft_workspace_size(const vg_shape *shape, int32_t n_q, int32_t max_k,
                                         int32_t max_tail, size_t *bytes) {
  if (!bytes || !valid_shape(shape) || n_q < 1 || max_k < 0 || max_tail < n_q)
    return VG_ERR_INVALID_ARG;
  const vg_status sup = supported_shape(shape);
  if (sup != VG_OK) return sup;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (n_q * G > kMaxRows) return VG_ERR_UNSUPPORTED;
  const AttnPlan p = plan_attention(shape, n_q, (long long)max_k + max_tail, true);
  if (!p.ok) return VG_ERR_UNSUPPORTED;
  *bytes = p.bytes;
  return VG_OK;
}

vg_status vg_sparse_draft_attention(const vg_shape *shape, const void *q, int32_t n_q,
                                    const void *k_cache, const void *v_cache,
                                    const int32_t *sel_slot, const int32_t *sel_count,
                                    int32_t max_k, const int32_t *page_table,
                                    const int32_t *tail_start, const int32_t *tail_len,
                                    int32_t max_tail, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return sparse_impl(shape, q, n_q, k_cache, v_cache, sel_slot, sel_count, max_k, page_table, tail_start,
                     tail_len, max_tail, out, workspace, workspace_bytes, stream);
}

vg_status vg_sparse_draft_attention_noalloc(const vg_shape *shape, const void *q, int32_t n_q,
                                            const void *k_cache, const void *v_cache,
                                            const int32_t *sel_slot, const int32_t *sel_count,
                                            int32_t max_k, const int32_t *page_table,
                                            const int32_t *tail_start, const int32_t *tail_len,
                                            int32_t max_tail, float *out, void *stream) {
  // The size check comes first: a call that needs more than the array holds
  // fails before anything touches the device.
  size_t need = 0;
  const vg_status q_st = vg_sparse_draft_workspace_size(shape, n_q, max_k, max_tail, &need);
  if (q_st != VG_OK) return q_st;
  if (need > kScratchBytes) return VG_ERR_WORKSPACE;
  void *ws = nullptr;
  const vg_status s_st = scratch_on_current_device(&ws);
  if (s_st != VG_OK) return s_st;
  return sparse_impl(shape, q, n_q, k_cache, v_cache, sel_slot, sel_count, max_k, page_table, tail_start,
                     tail_len, max_tail, out, ws, kScratchBytes, stream);
}

vg_status vg_kv_append(const vg_shape *shape, const void *k_new, const void *v_new, int32_t n_new,
                       const int32_t *page_table, const int32_t *start_pos, void *k_cache, void *v_cache,
                       void *stream) {
  if (!valid_shape(shape) || n_new < 0) return VG_ERR_INVALID_ARG;
  const void *req[] = {k_new, v_new, page_table, start_pos, k_cache, v_cache};
  for (const void *p : req)
    if (!p || !aligned16(p)) return VG_ERR_INVALID_ARG;
  const vg_status sup = supported_shape(shape);
  if (sup != VG_OK) return sup;
  if (n_new == 0) return VG_OK;
  if (n_new > 65535 || shape->batch > 65535) return VG_ERR_UNSUPPORTED;
  AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.start_pos = start_pos;
  a.n_new = n_new;
  a.max_pages = shape->max_pages_per_seq;
  const int elem = shape->dtype == VG_DTYPE_BF16 ? 2 : 4;
  a.row_vec16 = shape->num_kv_heads * shape->head_dim * elem / 16;
  hipLaunchKernelGGL(kv_append_kernel, dim3(n_new, shape->batch), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_window_select(int32_t batch, int32_t max_prefix, const int32_t *prefix_len, const int32_t *k,
                           int32_t max_k, int32_t n_sink, const int32_t *page_table, int32_t page_size,
                           int32_t max_pages_per_seq, int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count,
                           void *stream) {
  if (batch < 1 || batch > 65535 || max_prefix < 0 || max_k < 0 || n_sink < 0) return VG_ERR_INVALID_ARG;
  const void *req[] = {prefix_len, k, sel_pos, sel_count};
  for (const void *p : req)
    if (!p || !aligned16(p)) return VG_ERR_INVALID_ARG;
  if (sel_slot && (!aligned16(sel_slot) || !page_table || !aligned16(page_table) ||
                   page_size < 1 || max_pages_per_seq < 1 ||
                   ceil_div(max_prefix, page_size) > max_pages_per_seq))
    return VG_ERR_INVALID_ARG;
  WindowArgs a{};
  a.prefix_len = prefix_len;
  a.k = k;
  a.page_table = page_table;
  a.sel_pos = sel_pos;
  a.sel_slot = sel_slot;
  a.sel_count = sel_count;
  a.max_prefix = max_prefix;
  a.max_k = max_k;
  a.n_sink = n_sink;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  const int gx = std::max(1, std::min(ceil_div(max_k, 256), 64));
  hipLaunchKernelGGL(window_select_kernel, dim3(gx, batch), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

vg_status vg_advance_prefix(int32_t batch, int32_t gamma, const int32_t *n_accepted, int32_t *prefix_len,
                            void *stream) {
  if (batch < 0 || gamma < 0 || (batch > 0 && (!n_accepted || !prefix_len))) return VG_ERR_INVALID_ARG;
  if (batch == 0) return VG_OK;
  hipLaunchKernelGGL(advance_prefix_kernel, dim3((batch + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), batch, gamma, n_accepted, prefix_len);
  return hipGetLastError() == hipSuccess ? VG_OK : VG_ERR_HIP;
}

}  // extern "C"
