"""Device plumbing around the C-ABI: put a seeded workload in HBM, allocate
outputs and workspaces, and run the path's steps in order.

PyTorch is used only for device memory, streams and events; every step of
the path is a call into libvegas_attn.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _binding as vg
from .synth import Case


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)  # bf16 bit patterns travel as int16
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


# The V cache starts this many bytes into its own allocation, so that it sits
# 256 bytes past the K cache's (2 MB) alignment: same-head K and V rows then
# fall on different HBM channels (the cache placement note in vegas_attn.h).
V_CACHE_OFFSET = 256


def _v_cache(t: torch.Tensor) -> torch.Tensor:
    """A copy of the V cache t that starts V_CACHE_OFFSET bytes into its allocation."""
    buf = torch.empty(t.numel() * t.element_size() + V_CACHE_OFFSET, dtype=torch.uint8, device=t.device)
    v = buf[V_CACHE_OFFSET:].view(t.dtype).view(t.shape)
    v.copy_(t)
    return v


class DeviceCase:
    """One workload resident on the GPU, with every buffer the path writes."""

    def __init__(self, case: Case, device="cuda", kernel=vg.VG_KERNEL_AUTO, max_tail=None,
                 like: "DeviceCase | None" = None, pad=64):
        """`like`: another DeviceCase of the same workload whose inputs are copied on
        the device (a separate copy of the KV cache, e.g. another layer).
        `pad`: export / score rows are padded to a multiple of `pad` floats."""
        self.case = case
        self.device = torch.device(device)
        dev = self.device
        c = case
        self.B, self.Hq, self.Hkv, self.D = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim
        self.gamma, self.R = c.gamma, c.rows
        self.max_prefix, self.max_k = -(-max(c.max_prefix, 1) // pad) * pad, max(c.max_k, 1)
        self.dtype = vg.VG_DTYPE_BF16 if c.dtype == "bf16" else vg.VG_DTYPE_F32
        # room in the page-table rows for the padded max_prefix (entries past a
        # sequence's pages are -1 and never used)
        self.max_pages = max(c.max_pages, -(-(self.max_prefix + self.R) // c.page_size))
        self.shape = vg.make_shape(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                   self.max_pages, self.dtype, c.scale, kernel, c.page_size)
        if like is None:
            self.q = _dev(c.q, dev)
            self.q_draft = _dev(c.q_draft, dev)  # [gamma][B][Hq][D]
            self.k_cache = _dev(c.k_cache, dev)
            self.v_cache = _v_cache(_dev(c.v_cache, dev))
            pt = np.full((c.batch, self.max_pages), -1, dtype=np.int32)
            pt[:, : c.max_pages] = c.page_table
            self.page_table = _dev(pt, dev)
            self.prefix_len = _dev(c.prefix_len, dev)
            self.k = _dev(c.k, dev)
        else:
            for n in ("q", "q_draft", "k_cache", "page_table", "prefix_len"):
                setattr(self, n, getattr(like, n).clone())
            self.v_cache = _v_cache(like.v_cache)
            self.k = _dev(c.k, dev)  # the budget may differ (same inputs, another k)
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        mp = self.max_prefix
        self.out = torch.zeros(self.B, self.R, self.Hq, self.D, **f32)
        self.logits = torch.zeros(self.B, 2, self.Hq, mp, **f32)
        self.group = torch.zeros(self.B, self.Hkv, mp, **f32)
        self.scores = torch.zeros(self.B, mp, **f32)
        self.sel_pos = torch.full((self.B, self.max_k), -1, **i32)
        self.sel_slot = torch.full((self.B, self.max_k), -1, **i32)
        self.sel_count = torch.zeros(self.B, **i32)
        self.draft_out = torch.zeros(self.B, 1, self.Hq, self.D, **f32)
        self.tail_start = self.prefix_len.clone()
        self.max_tail = int(max_tail) if max_tail is not None else self.R
        self.tail_len = [torch.full((self.B,), s + 1, **i32) for s in range(max(self.gamma, 1))]
        self.ws_verify_bytes = vg.vg_verify_workspace_size(self.shape, self.max_prefix, self.gamma)
        self.ws_select_bytes = vg.vg_topk_workspace_size(self.B, self.max_prefix)
        self.ws_sparse_bytes = vg.vg_sparse_draft_workspace_size(self.shape, 1, self.max_k, self.max_tail)
        self.ws_verify = self._workspace(self.ws_verify_bytes)
        self.ws_select = self._workspace(self.ws_select_bytes)
        self.ws_sparse = self._workspace(self.ws_sparse_bytes)

    def _workspace(self, nbytes):
        ws = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=self.device)
        vg.vg_workspace_zero(ws, ws.numel())
        return ws

    # ------------------------------------------------------------------ steps
    @property
    def logits_all(self):
        """Every verify row's logits [B][R][Hq][max_prefix] (full collection), allocated on first use."""
        if getattr(self, "_logits_all", None) is None:
            self._logits_all = torch.zeros(self.B, self.R, self.Hq, self.max_prefix, dtype=torch.float32,
                                           device=self.device)
        return self._logits_all

    def verify(self, export="both", rows="two", stream=None):
        """export: "raw", "group", "both" or "none"; rows: "two" (Collect-2-Query: rows 0
        and gamma into `logits`) or "all" (every row into `logits_all`; `group` then sums
        all rows)."""
        raw = self.logits if rows == "two" else self.logits_all
        logits = raw if export in ("raw", "both") else None
        group = self.group if export in ("group", "both") else None
        fn = vg.vg_verify_attention if rows == "two" else vg.vg_verify_attention_all_rows
        fn(self.shape, self.q, self.k_cache, self.v_cache, self.page_table, self.prefix_len, self.max_prefix,
           self.gamma, self.out, logits, group, self.ws_verify, self.ws_verify_bytes, stream)

    def _export(self, src):
        """(buffer, rows, heads) of an export: "raw" (two rows), "raw_all" (every row) or "group"."""
        if src == "raw":
            return self.logits, 2, self.Hq
        if src == "raw_all":
            return self.logits_all, self.R, self.Hq
        return self.group, 1, self.Hkv

    def aggregate(self, src="raw", fuse_prepass=False, stream=None):
        """src: "raw" (two rows), "raw_all" (every row) or "group"."""
        t, rows, heads = self._export(src)
        ws = self.ws_select if fuse_prepass else None
        vg.vg_aggregate_scores(self.B, t, rows, heads, self.prefix_len, self.max_prefix, self.scores,
                               ws, self.ws_select_bytes if fuse_prepass else 0, stream)

    def topk(self, scores=None, prepass_done=False, stream=None):
        flags = vg.VG_TOPK_PREPASS_DONE if prepass_done else 0
        vg.vg_topk_select(self.B, self.scores if scores is None else scores, self.max_prefix,
                          self.prefix_len, self.k, self.max_k, self.page_table, self.case.page_size,
                          self.max_pages, self.sel_pos, self.sel_slot, self.sel_count, flags,
                          self.ws_select, self.ws_select_bytes, stream)

    def select(self, src="group", stream=None):
        """Aggregation and top-k in one call (vg_aggregate_topk_select): scores, then
        the selection into sel_pos / sel_slot / sel_count.  src as for aggregate()."""
        t, rows, heads = self._export(src)
        vg.vg_aggregate_topk_select(self.B, t, rows, heads, self.prefix_len, self.max_prefix, self.scores,
                                    self.k, self.max_k, self.page_table, self.case.page_size, self.max_pages,
                                    self.sel_pos, self.sel_slot, self.sel_count, self.ws_select,
                                    self.ws_select_bytes, stream)

    def verify_select(self, stream=None):
        """Verify with the group export, aggregation and top-k in one call (vg_verify_select)."""
        vg.vg_verify_select(self.shape, self.q, self.k_cache, self.v_cache, self.page_table, self.prefix_len,
                            self.max_prefix, self.gamma, self.out, self.group, self.scores, self.k, self.max_k,
                            self.sel_pos, self.sel_slot, self.sel_count, self.ws_verify, self.ws_verify_bytes,
                            self.ws_select, self.ws_select_bytes, stream)

    def window(self, n_sink=4, stream=None):
        """Query-agnostic selection into the same buffers as topk(): n_sink sink
        positions plus the most recent ones, k_b in all."""
        vg.vg_window_select(self.B, self.max_prefix, self.prefix_len, self.k, self.max_k, n_sink,
                            self.page_table, self.case.page_size, self.max_pages, self.sel_pos,
                            self.sel_slot, self.sel_count, stream)

    def sparse(self, step=0, q=None, sel_slot=None, sel_count=None, tail_start=None, tail_len=None,
               out=None, n_q=1, stream=None):
        qq = self.q_draft[step] if q is None else q
        vg.vg_sparse_draft_attention(
            self.shape, qq, n_q, self.k_cache, self.v_cache,
            self.sel_slot if sel_slot is None else sel_slot,
            self.sel_count if sel_count is None else sel_count,
            self.max_k, self.page_table,
            self.tail_start if tail_start is None else tail_start,
            self.tail_len[step] if tail_len is None else tail_len,
            self.max_tail, self.draft_out if out is None else out,
            self.ws_sparse, self.ws_sparse_bytes, stream)

    def new_rows(self):
        """The R new tokens' K/V rows [B][R][Hkv][D] as generated (copies of their
        cache rows), on the device: an append of these rewrites the same values."""
        if getattr(self, "_new_rows", None) is None:
            c, ps = self.case, self.case.page_size
            p = c.prefix_len.astype(np.int64)[:, None] + np.arange(self.R)
            slot = c.page_table[np.arange(self.B)[:, None], p // ps].astype(np.int64) * ps + p % ps
            idx = torch.from_numpy(slot.reshape(-1)).to(self.device)
            shp = (self.B, self.R, self.Hkv, self.D)
            self._new_rows = (self.k_cache[idx].reshape(shp).contiguous(),
                              self.v_cache[idx].reshape(shp).contiguous())
        return self._new_rows

    def append(self, k_new=None, v_new=None, start_pos=None, stream=None):
        """Write the new tokens' rows at positions start_pos[b] + r (default: prefix_len)."""
        if k_new is None:
            k_new, v_new = self.new_rows()
        vg.vg_kv_append(self.shape, k_new, v_new, k_new.shape[1], self.page_table,
                        self.prefix_len if start_pos is None else start_pos, self.k_cache, self.v_cache, stream)

    def advance(self, n_accepted, stream=None):
        """Keep the first new token and the accepted drafts: prefix_len += 1 + n."""
        vg.vg_advance_prefix(self.B, self.gamma, n_accepted, self.prefix_len, stream)

    def iteration(self, export="group", rows="two", stream=None):
        """One pass of the whole path: verify (+export), aggregate, top-k, gamma draft steps."""
        if export == "group" and rows == "two":
            self.verify_select(stream=stream)
        else:
            self.verify(export=export, rows=rows, stream=stream)
            self.select(src="raw" if rows == "two" else "raw_all", stream=stream)
        for s in range(self.gamma):
            self.sparse(step=s, stream=stream)

    # ------------------------------------------------------------- host copies
    _PADDED = ("logits", "logits_all", "group", "scores")  # last dim padded past the case's max_prefix

    def host(self, name):
        """Host copy of a device buffer (padded rows trimmed to the case's max_prefix)."""
        a = getattr(self, name).detach().cpu().numpy()
        if name in self._PADDED:
            a = a[..., : self.case.max_prefix]
        return a

    def put(self, name, array):
        """Copy a host array into the leading part of a device buffer."""
        import torch
        t = torch.from_numpy(np.ascontiguousarray(array))
        dst = getattr(self, name)
        if name in self._PADDED:
            dst[..., : t.shape[-1]].copy_(t)
        else:
            dst.copy_(t)
