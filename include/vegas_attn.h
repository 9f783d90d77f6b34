/*
 * vegas_attn.h -- C-ABI of the MI355X (gfx950) hot path of Vegas's
 * verification-guided sparse attention, one decode iteration of one layer:
 *
 *   vg_verify_attention        full causal attention of the gamma+1 verify
 *                              rows over the whole paged KV cache, exporting
 *                              the pre-softmax logits of row 0 (first draft
 *                              token) and row gamma (bonus token).
 *   vg_aggregate_scores        one score per prefix position: the exported
 *                              logits summed over rows and query heads.
 *   vg_topk_select             the k prefix positions with the largest
 *                              scores, as ascending positions and as
 *                              page-size-1 slot ids.
 *   vg_sparse_draft_attention  attention of draft rows over only the selected
 *                              slots plus the causal tail after the prefix.
 *
 * Fused forms of the same steps: vg_aggregate_topk_select (aggregation and
 * top-k in one call) and vg_verify_select (verify with the group export,
 * aggregation and top-k in one call).  Around the path: the all-rows export
 * (vg_verify_attention_all_rows), the KV append and prefix bookkeeping
 * (vg_kv_append, vg_advance_prefix), a query-agnostic selector
 * (vg_window_select), and a draft call that allocates nothing
 * (vg_sparse_draft_attention_noalloc).
 *
 * "Vegas" below is the page "Vegas: Self-Speculative Decoding with
 * Verification-Guided Sparse Attention" (technical summary).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   allocates nothing, keeps no per-call state between calls except inside
 *   the caller's workspace (and, for vg_sparse_draft_attention_noalloc only,
 *   its file-scope scratch array), and never synchronises the stream or
 *   copies device data to the host.  Work is enqueued on `stream` (a hipStream_t
 *   passed as void*; NULL = the null stream).
 * - Arguments are validated on the host before anything is enqueued.  On any
 *   error nothing is launched and no output is touched.  Values that live on
 *   the device (prefix lengths, k, page-table entries, slot ids) cannot be
 *   checked without a synchronisation; their preconditions are stated per
 *   call, and violating them is undefined behaviour.
 * - Device pointers must be 16-byte aligned.
 * - Workspaces: sized by the matching *_workspace_size query, and zero-filled
 *   once before first use (vg_workspace_zero does it).  Every call leaves its
 *   workspace zero-filled again where it needs zeros, so a workspace can be
 *   reused by later calls on the same stream; it must not be shared by calls
 *   that may run concurrently.
 * - KV cache layout: token-major paged cache, element [slot][kv_head][d] with
 *   slot = page * page_size + offset, i.e. [num_pages][page_size][Hkv][D].
 *   A slot id is the index of a page of one token (Vegas section 3, sparse
 *   execution: selected token indices are passed as page indices of a
 *   page-size-1 PagedAttention call).
 *   Placement (performance only; any 16-byte aligned bases work): give the V
 *   cache a base 256 bytes past the alignment of the K cache's base (for
 *   example both from 2 MB-aligned allocations, V starting 256 bytes in).
 *   The kernels read the K and V rows of a head together; with equally
 *   aligned bases those rows have the same low address bits and load the
 *   same HBM channels.  Measured on MI355X: the 128K verify call without
 *   export 97 -> 93.5 us, the batch-8 ragged one 404 -> 383 us.
 * - Query head h uses KV head h / (Hq / Hkv).
 * - Outputs are fp32.
 */
#ifndef VEGAS_ATTN_H
#define VEGAS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vg_status;
#define VG_OK 0
#define VG_ERR_INVALID_ARG 1  /* a null/misaligned pointer or an out-of-range argument */
#define VG_ERR_UNSUPPORTED 2  /* a valid shape the library has no kernel for */
#define VG_ERR_WORKSPACE 3    /* workspace missing or smaller than the size query says */
#define VG_ERR_HIP 4          /* the HIP runtime rejected a launch */

#define VG_DTYPE_F32 0
#define VG_DTYPE_BF16 1

#define VG_KERNEL_AUTO 0 /* MFMA for bf16, VALU for f32 */
#define VG_KERNEL_VALU 1 /* vector-ALU contraction (f32 and bf16) */
#define VG_KERNEL_MFMA 2 /* matrix-core contraction (bf16 only) */

/* Shape of one attention layer and its paged cache. */
typedef struct vg_shape {
  int32_t batch;             /* B >= 1 sequences; attention calls take B <= 1024
                                (more gives VG_ERR_UNSUPPORTED) */
  int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t page_size;         /* tokens per page: 16 */
  int32_t max_pages_per_seq; /* row length of page_table */
  int32_t dtype;             /* VG_DTYPE_*: element type of q, k_cache, v_cache */
  float softmax_scale;       /* logit = softmax_scale * q.k; <= 0 selects 1/sqrt(D) */
  int32_t kernel;            /* VG_KERNEL_* */
} vg_shape;

/* Human-readable name of a status code (static string). */
const char *vg_status_string(vg_status status);

/* Library version string (static). */
const char *vg_version(void);

/* Zero-fill `bytes` of device workspace on `stream` (a kernel, no memset node). */
vg_status vg_workspace_zero(void *workspace, size_t bytes, void *stream);

/* ---------------------------------------------------------------- verify */

/* Workspace bytes vg_verify_attention needs for this shape and these maxima. */
vg_status vg_verify_workspace_size(const vg_shape *shape, int32_t max_prefix, int32_t gamma,
                                   size_t *bytes);

/*
 * Verification attention with the Collect-2-Query logit export.
 *
 * Vegas section 2 (core mechanism, verification phase): verification is a
 * standard full-attention pass that computes the attention logits of every KV
 * entry.  Section 2.B (Collect-2-Query): only the first draft token and the
 * bonus token export their logits.  Section 3 (kernel instrumentation): the
 * logits are written to HBM before softmax normalisation.
 *
 * For each sequence b with prefix length P_b = prefix_len[b], the cache holds
 * N_b = P_b + gamma + 1 tokens at logical positions 0..N_b-1 (the gamma+1 new
 * tokens already appended at P_b..P_b+gamma).  Row r in [0, gamma] attends
 * causally to positions 0..P_b+r:
 *     l[r][h][j] = scale * q[b][r][h] . K[b][j][h/G]
 *     out[b][r][h] = sum_j softmax_j(l[r][h][.]) V[b][j][h/G]
 *
 *   q            [B][gamma+1][Hq][D]  dtype
 *   k_cache      [num_slots][Hkv][D]  dtype
 *   v_cache      [num_slots][Hkv][D]  dtype
 *   page_table   [B][max_pages_per_seq] int32: logical page -> physical page
 *   prefix_len   [B] int32, 0 <= P_b <= max_prefix, and
 *                ceil((P_b+gamma+1)/page_size) <= max_pages_per_seq
 *   gamma        0 <= gamma <= 15 (draft tokens; gamma+1 verify rows)
 *   out          [B][gamma+1][Hq][D] float (written)
 *   logits       [B][2][Hq][max_prefix] float, nullable: [b][0][h][j] = l[0][h][j],
 *                [b][1][h][j] = l[gamma][h][j] for j < P_b (natural-log units,
 *                scale applied); entries j >= P_b are not written.
 *   group_scores [B][Hkv][max_prefix] float, nullable: sum over the G query
 *                heads of KV head g of both exported rows, for j < P_b.
 *   Both exports may be null (plain causal attention, no export).
 * Supported: D in {64, 128}; page_size 16; (gamma+1)*G <= 64; bf16 with any
 * kernel, f32 with VG_KERNEL_VALU or AUTO.
 */
vg_status vg_verify_attention(const vg_shape *shape, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *page_table,
                              const int32_t *prefix_len, int32_t max_prefix, int32_t gamma,
                              float *out, float *logits, float *group_scores, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Verification attention with the full-collection logit export: the logits of
 * every verify row, i.e. the selection objective of Vegas section 2.A summed
 * over all gamma+1 verify tokens, which Collect-2-Query (section 2.B) reduces
 * to two rows.  Provided to measure that reduction.
 *
 * Same arguments, preconditions, workspace (vg_verify_workspace_size) and
 * errors as vg_verify_attention, except the exports:
 *   logits       [B][gamma+1][Hq][max_prefix] float, nullable: [b][r][h][j] =
 *                l[r][h][j] for j < P_b; entries j >= P_b are not written.
 *   group_scores [B][Hkv][max_prefix] float, nullable: sum over all gamma+1
 *                rows and the G query heads of KV head g, for j < P_b.
 * vg_aggregate_scores with src_rows = gamma+1 turns the raw form into scores.
 */
vg_status vg_verify_attention_all_rows(const vg_shape *shape, const void *q, const void *k_cache,
                                       const void *v_cache, const int32_t *page_table,
                                       const int32_t *prefix_len, int32_t max_prefix, int32_t gamma,
                                       float *out, float *logits, float *group_scores,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------- aggregate */

/*
 * Score of each prefix position (Vegas section 2.A, selection objective,
 * restricted by section 2.B to the exported rows):
 *     scores[b][j] = sum_{t < src_rows} sum_{h < src_heads} src[b][t][h][j],  j < P_b.
 * Use src = logits with (src_rows, src_heads) = (2, Hq), or src = group_scores
 * with (1, Hkv).  Entries j >= P_b of `scores` are not written.
 *
 *   src         [B][src_rows][src_heads][max_prefix] float
 *   prefix_len  [B] int32, 0 <= P_b <= max_prefix
 *   scores      [B][max_prefix] float (written)
 *   select_ws   nullable.  A vg_topk_select workspace sized for (batch,
 *               max_prefix).  When given, the first pass of the top-k
 *               selection over the new scores is fused into this call and its
 *               result kept in select_ws; pass VG_TOPK_PREPASS_DONE to the next
 *               vg_topk_select on the same scores and workspace.
 */
vg_status vg_aggregate_scores(int32_t batch, const float *src, int32_t src_rows, int32_t src_heads,
                              const int32_t *prefix_len, int32_t max_prefix, float *scores,
                              void *select_ws, size_t select_ws_bytes, void *stream);

/* ------------------------------------------------------------------ topk */

#define VG_TOPK_PREPASS_DONE 1 /* vg_aggregate_scores already ran the first pass */

/* Workspace bytes vg_topk_select (and a fused vg_aggregate_scores) needs. */
vg_status vg_topk_workspace_size(int32_t batch, int32_t max_prefix, size_t *bytes);

/*
 * Exact top-k selection (Vegas section 2.A: T maximises the summed score over
 * all subsets of k prefix positions; the sum is additive over positions, so T
 * is the set of the k largest scores).
 *
 * For each b, with kk = min(k[b], P_b): writes the kk positions j < P_b with
 * the largest scores[b][j], ascending, to sel_pos[b][0..kk); equal scores at
 * the threshold are taken lowest position first (-0.0 counts as +0.0);
 * sel_count[b] = kk.  sel_slot (nullable) receives the page-size-1 slot of
 * each position: page_table[b][pos / page_size] * page_size + pos % page_size.
 * Entries past kk are not written.  Scores must be finite.
 *
 *   scores      [B][max_prefix] float
 *   prefix_len  [B] int32, 0 <= P_b <= max_prefix
 *   k           [B] int32, 0 <= k[b] <= max_k
 *   page_table  [B][max_pages_per_seq] int32 (needed when sel_slot is non-null)
 *   sel_pos     [B][max_k] int32;  sel_slot [B][max_k] int32;  sel_count [B] int32
 *   flags       0 or VG_TOPK_PREPASS_DONE
 */
vg_status vg_topk_select(int32_t batch, const float *scores, int32_t max_prefix,
                         const int32_t *prefix_len, const int32_t *k, int32_t max_k,
                         const int32_t *page_table, int32_t page_size, int32_t max_pages_per_seq,
                         int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count, int32_t flags,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Aggregation and exact top-k selection in one call: vg_aggregate_scores
 * (scores from the exported logits, Vegas section 2.A objective restricted by
 * section 2.B to the exported rows) followed by vg_topk_select (section 2.A:
 * the k largest scores), with the same results as that pair of calls.
 *
 *   src, src_rows, src_heads, prefix_len, max_prefix, scores: as for
 *       vg_aggregate_scores (scores[b][j] is written for j < P_b);
 *   k, max_k, page_table, page_size, max_pages_per_seq, sel_pos, sel_slot,
 *       sel_count: as for vg_topk_select;
 *   workspace: sized by vg_topk_workspace_size(batch, max_prefix), zero-filled
 *       once before first use (the call leaves it zero-filled again).
 * With max_prefix <= 131072 and even, and page_size 16 (or sel_slot null), the
 * selection runs in two kernel launches (per-chunk staging, then the exact
 * threshold and the output); otherwise in three (radix passes).
 */
vg_status vg_aggregate_topk_select(int32_t batch, const float *src, int32_t src_rows, int32_t src_heads,
                                   const int32_t *prefix_len, int32_t max_prefix, float *scores,
                                   const int32_t *k, int32_t max_k, const int32_t *page_table,
                                   int32_t page_size, int32_t max_pages_per_seq, int32_t *sel_pos,
                                   int32_t *sel_slot, int32_t *sel_count, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Verification attention with the group export, then aggregation and exact
 * top-k selection (Vegas section 2: verification computes every entry's
 * logits; section 2.B: the first draft token's and the bonus token's are
 * collected; section 2.A: the k positions with the largest summed logits are
 * selected), with the same results as
 *     vg_verify_attention(..., logits = NULL, group_scores, ...)
 *     vg_aggregate_topk_select(batch, group_scores, 1, Hkv, prefix_len, max_prefix, scores, ...).
 * The selection's first step runs in the same launch as the verify combine.
 *
 *   shape .. out, verify_ws: as for vg_verify_attention (group_scores must be
 *       non-null; raw logits are not exported);
 *   scores, k, max_k, sel_pos, sel_slot, sel_count: as for
 *       vg_aggregate_topk_select, with page_table, page_size and
 *       max_pages_per_seq taken from the verify arguments;
 *   select_ws: sized by vg_topk_workspace_size(batch, max_prefix), zero-filled
 *       once before first use.
 */
vg_status vg_verify_select(const vg_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *page_table, const int32_t *prefix_len, int32_t max_prefix, int32_t gamma,
                           float *out, float *group_scores, float *scores, const int32_t *k, int32_t max_k,
                           int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count, void *verify_ws,
                           size_t verify_ws_bytes, void *select_ws, size_t select_ws_bytes, void *stream);

/* --------------------------------------------------------- sparse draft */

/* Workspace bytes vg_sparse_draft_attention needs. */
vg_status vg_sparse_draft_workspace_size(const vg_shape *shape, int32_t n_q, int32_t max_k,
                                         int32_t max_tail, size_t *bytes);

/*
 * Sparse draft attention (Vegas section 2, core mechanism, drafting phase:
 * attention restricted to the selected critical entries; section 3, sparse
 * execution: the selected token indices are the pages of a page-size-1
 * PagedAttention call).
 *
 * Row i in [0, n_q) of sequence b attends to the key list
 *     sel_slot[b][0..cnt)  ++  slots of positions tail_start[b] .. tail_start[b]+tail_len[b]-n_q+i
 * (cnt = sel_count[b]; tail positions translated through page_table):
 *     out[b][i][h] = sum over the list of softmax(scale * q.K) V  (KV head h/G).
 *
 *   q          [B][n_q][Hq][D] dtype, 1 <= n_q and n_q * G <= 64
 *   sel_slot   [B][max_k] int32 slot ids (as written by vg_topk_select)
 *   sel_count  [B] int32, 0 <= cnt <= max_k
 *   page_table [B][max_pages_per_seq] int32
 *   tail_start [B] int32 >= 0;  tail_len [B] int32 with n_q <= tail_len <= max_tail,
 *              every tail position within the sequence's pages
 *   max_tail   host-side bound on tail_len, n_q <= max_tail
 *   out        [B][n_q][Hq][D] float (written)
 */
vg_status vg_sparse_draft_attention(const vg_shape *shape, const void *q, int32_t n_q,
                                    const void *k_cache, const void *v_cache,
                                    const int32_t *sel_slot, const int32_t *sel_count,
                                    int32_t max_k, const int32_t *page_table,
                                    const int32_t *tail_start, const int32_t *tail_len,
                                    int32_t max_tail, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as vg_sparse_draft_attention, with the same arguments except the
 * workspace, which is a device array built into the library instead of a
 * caller-provided buffer.
 *
 * The array is VG_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held from the
 * library's load until the process ends.  A call whose
 * vg_sparse_draft_workspace_size exceeds it returns VG_ERR_WORKSPACE and
 * launches nothing.  Nothing in this call allocates (no hipMalloc, hipFree
 * or allocating library routine); its first call on a device looks up the
 * array's device address (hipGetSymbolAddress) and keeps it for later calls.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * partial results: calls that may overlap on one GPU (different streams,
 * concurrent host threads) race and must be ordered by the caller.  The
 * array needs no zero state.  Results are bit-identical to
 * vg_sparse_draft_attention's for the same inputs.
 */
#define VG_NOALLOC_SCRATCH_BYTES (8u << 20)
vg_status vg_sparse_draft_attention_noalloc(const vg_shape *shape, const void *q, int32_t n_q,
                                            const void *k_cache, const void *v_cache,
                                            const int32_t *sel_slot, const int32_t *sel_count,
                                            int32_t max_k, const int32_t *page_table,
                                            const int32_t *tail_start, const int32_t *tail_len,
                                            int32_t max_tail, float *out, void *stream);

/*
 * Query-agnostic selection (Vegas section 1: sliding-window style selection
 * has little overhead but drafts less accurately; section 4 compares against
 * such a streaming baseline): the first n_sink prefix positions (attention
 * sinks) and the most recent ones, k_b positions in all, in the same output
 * form as vg_topk_select, so that vg_sparse_draft_attention takes either list.
 * With kk = min(k[b], P_b, max_k) and s = min(n_sink, kk):
 *     sel_pos[b][0..kk) = 0, 1, ..., s-1, P_b-(kk-s), ..., P_b-1   (ascending)
 *     sel_slot[b][i]    = page_table[b][pos / page_size] * page_size + pos % page_size
 *     sel_count[b]      = kk
 * Entries past kk are not written.  No scores are read.
 *
 *   prefix_len  [B] int32, 0 <= P_b <= max_prefix (clamped to that range)
 *   k           [B] int32, 0 <= k[b] <= max_k (clamped)
 *   n_sink      >= 0
 *   page_table  [B][max_pages_per_seq] int32 (needed when sel_slot is non-null)
 *   sel_pos     [B][max_k] int32;  sel_slot [B][max_k] int32 (nullable);  sel_count [B] int32
 * 1 <= batch <= 65535.
 */
vg_status vg_window_select(int32_t batch, int32_t max_prefix, const int32_t *prefix_len, const int32_t *k,
                           int32_t max_k, int32_t n_sink, const int32_t *page_table, int32_t page_size,
                           int32_t max_pages_per_seq, int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count,
                           void *stream);

/* ------------------------------------------------------------- KV append */

/*
 * Append the new tokens' K/V rows to the paged cache: the step before
 * verification (the gamma+1 tokens verify attends to must already be cached;
 * Vegas section 2, core mechanism), so that a whole iteration runs on the
 * device.  For every sequence b, new token r in [0, n_new) and KV head g:
 *     k_cache[slot(b, start_pos[b] + r)][g][:] = k_new[b][r][g][:]   (same for V)
 * with slot(b, pos) = page_table[b][pos / 16] * 16 + pos % 16.  Copies are exact.
 *
 *   k_new, v_new  [B][n_new][Hkv][D] dtype (read)
 *   page_table    [B][max_pages_per_seq] int32
 *   start_pos     [B] int32: logical position of new token 0 (P_b for verify)
 *   k_cache, v_cache [num_slots][Hkv][D] dtype (written at the new tokens' slots only)
 *   n_new         0 <= n_new <= 65535 (0: nothing launched)
 * Positions whose page-table entry is outside the row or negative are skipped.
 * Supported: D in {64, 128}; page_size 16; f32 or bf16.
 */
vg_status vg_kv_append(const vg_shape *shape, const void *k_new, const void *v_new, int32_t n_new,
                       const int32_t *page_table, const int32_t *start_pos, void *k_cache, void *v_cache,
                       void *stream);

/*
 * Tail bookkeeping between iterations.  Of an iteration's gamma + 1 new tokens
 * the sequence keeps the first (the token carried over from the previous
 * iteration) and the n_accepted[b] draft tokens that verification accepted;
 * the rejected drafts' slots are overwritten by the next append (Vegas
 * section 2: drafts are accepted or rejected by verification):
 *     prefix_len[b] += 1 + min(max(n_accepted[b], 0), gamma)
 *
 *   n_accepted  [B] int32 device (read)
 *   prefix_len  [B] int32 device (updated in place)
 * Pages for the grown sequences must already be in the page table (page
 * allocation is the caller's).  batch = 0 launches nothing.
 */
vg_status vg_advance_prefix(int32_t batch, int32_t gamma, const int32_t *n_accepted, int32_t *prefix_len,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VEGAS_ATTN_H */
