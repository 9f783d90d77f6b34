"""ctypes binding of libvegas_attn.so (the C-ABI in include/vegas_attn.h).

Argument marshalling only: torch tensors are passed as raw device pointers,
every step of the path runs in the library's HIP kernels.  The functions keep
the C names; a non-VG_OK status raises VgError.  If the library is missing,
loading fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("VG_LIB_PATH") or os.path.join(_HERE, "libvegas_attn.so")

VG_OK = 0
VG_ERR_INVALID_ARG = 1
VG_ERR_UNSUPPORTED = 2
VG_ERR_WORKSPACE = 3
VG_ERR_HIP = 4

VG_DTYPE_F32 = 0
VG_DTYPE_BF16 = 1

VG_KERNEL_AUTO = 0
VG_KERNEL_VALU = 1
VG_KERNEL_MFMA = 2

VG_TOPK_PREPASS_DONE = 1

VG_NOALLOC_SCRATCH_BYTES = 8 << 20  # the built-in workspace of vg_sparse_draft_attention_noalloc

# every symbol include/vegas_attn.h declares
EXPORTS = (
    "vg_status_string", "vg_version", "vg_workspace_zero",
    "vg_verify_workspace_size", "vg_verify_attention", "vg_verify_attention_all_rows",
    "vg_aggregate_scores",
    "vg_topk_workspace_size", "vg_topk_select", "vg_aggregate_topk_select", "vg_verify_select",
    "vg_sparse_draft_workspace_size", "vg_sparse_draft_attention", "vg_sparse_draft_attention_noalloc",
    "vg_window_select", "vg_kv_append", "vg_advance_prefix",
)


class VgError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class VgShape(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("page_size", C.c_int32),
        ("max_pages_per_seq", C.c_int32),
        ("dtype", C.c_int32),
        ("softmax_scale", C.c_float),
        ("kernel", C.c_int32),
    ]


_lib = None


def lib():
    """Load libvegas_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m verification_guided_sparse_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
        SP = C.POINTER(VgShape)
        L.vg_status_string.argtypes = [I32]
        L.vg_status_string.restype = C.c_char_p
        L.vg_version.argtypes = []
        L.vg_version.restype = C.c_char_p
        L.vg_workspace_zero.argtypes = [P, SZ, P]
        L.vg_verify_workspace_size.argtypes = [SP, I32, I32, C.POINTER(SZ)]
        L.vg_verify_attention.argtypes = [SP, P, P, P, P, P, I32, I32, P, P, P, P, SZ, P]
        L.vg_verify_attention_all_rows.argtypes = [SP, P, P, P, P, P, I32, I32, P, P, P, P, SZ, P]
        L.vg_aggregate_scores.argtypes = [I32, P, I32, I32, P, I32, P, P, SZ, P]
        L.vg_topk_workspace_size.argtypes = [I32, I32, C.POINTER(SZ)]
        L.vg_topk_select.argtypes = [I32, P, I32, P, P, I32, P, I32, I32, P, P, P, I32, P, SZ, P]
        L.vg_verify_select.argtypes = [SP, P, P, P, P, P, I32, I32, P, P, P, P, I32, P, P, P, P, SZ, P, SZ, P]
        L.vg_aggregate_topk_select.argtypes = [I32, P, I32, I32, P, I32, P, P, I32, P, I32, I32, P, P, P, P,
                                               SZ, P]
        L.vg_sparse_draft_workspace_size.argtypes = [SP, I32, I32, I32, C.POINTER(SZ)]
        L.vg_sparse_draft_attention.argtypes = [SP, P, I32, P, P, P, P, I32, P, P, P, I32, P, P, SZ, P]
        L.vg_sparse_draft_attention_noalloc.argtypes = [SP, P, I32, P, P, P, P, I32, P, P, P, I32, P, P]
        L.vg_window_select.argtypes = [I32, I32, P, P, I32, I32, P, I32, I32, P, P, P, P]
        L.vg_kv_append.argtypes = [SP, P, P, I32, P, P, P, P, P]
        L.vg_advance_prefix.argtypes = [I32, I32, P, P, P]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().vg_status_string(int(status)).decode()


def version() -> str:
    return lib().vg_version().decode()


def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != VG_OK:
        raise VgError(fn, status)


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq, dtype,
               softmax_scale=0.0, kernel=VG_KERNEL_AUTO, page_size=16) -> VgShape:
    return VgShape(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                   int(max_pages_per_seq), int(dtype), float(softmax_scale), int(kernel))


def vg_workspace_zero(workspace, nbytes, stream=None):
    _check("vg_workspace_zero", lib().vg_workspace_zero(_ptr(workspace), int(nbytes), _stream(stream)))


def vg_verify_workspace_size(shape: VgShape, max_prefix: int, gamma: int) -> int:
    n = C.c_size_t(0)
    _check("vg_verify_workspace_size",
           lib().vg_verify_workspace_size(C.byref(shape), int(max_prefix), int(gamma), C.byref(n)))
    return n.value


def vg_verify_attention(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma, out,
                        logits, group_scores, workspace, workspace_bytes, stream=None):
    _check("vg_verify_attention", lib().vg_verify_attention(
        C.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(prefix_len),
        int(max_prefix), int(gamma), _ptr(out), _ptr(logits), _ptr(group_scores), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def vg_verify_attention_all_rows(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma,
                                 out, logits, group_scores, workspace, workspace_bytes, stream=None):
    _check("vg_verify_attention_all_rows", lib().vg_verify_attention_all_rows(
        C.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(prefix_len),
        int(max_prefix), int(gamma), _ptr(out), _ptr(logits), _ptr(group_scores), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def vg_aggregate_scores(batch, src, src_rows, src_heads, prefix_len, max_prefix, scores,
                        select_ws=None, select_ws_bytes=0, stream=None):
    _check("vg_aggregate_scores", lib().vg_aggregate_scores(
        int(batch), _ptr(src), int(src_rows), int(src_heads), _ptr(prefix_len), int(max_prefix),
        _ptr(scores), _ptr(select_ws), int(select_ws_bytes), _stream(stream)))


def vg_topk_workspace_size(batch: int, max_prefix: int) -> int:
    n = C.c_size_t(0)
    _check("vg_topk_workspace_size", lib().vg_topk_workspace_size(int(batch), int(max_prefix), C.byref(n)))
    return n.value


def vg_topk_select(batch, scores, max_prefix, prefix_len, k, max_k, page_table, page_size,
                   max_pages_per_seq, sel_pos, sel_slot, sel_count, flags, workspace,
                   workspace_bytes, stream=None):
    _check("vg_topk_select", lib().vg_topk_select(
        int(batch), _ptr(scores), int(max_prefix), _ptr(prefix_len), _ptr(k), int(max_k),
        _ptr(page_table), int(page_size), int(max_pages_per_seq), _ptr(sel_pos), _ptr(sel_slot),
        _ptr(sel_count), int(flags), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def vg_aggregate_topk_select(batch, src, src_rows, src_heads, prefix_len, max_prefix, scores, k, max_k,
                             page_table, page_size, max_pages, sel_pos, sel_slot, sel_count, workspace,
                             workspace_bytes, stream=None):
    _check("vg_aggregate_topk_select", lib().vg_aggregate_topk_select(
        int(batch), _ptr(src), int(src_rows), int(src_heads), _ptr(prefix_len), int(max_prefix), _ptr(scores),
        _ptr(k), int(max_k), _ptr(page_table), int(page_size), int(max_pages), _ptr(sel_pos), _ptr(sel_slot),
        _ptr(sel_count), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def vg_verify_select(shape, q, k_cache, v_cache, page_table, prefix_len, max_prefix, gamma, out, group_scores,
                     scores, k, max_k, sel_pos, sel_slot, sel_count, verify_ws, verify_ws_bytes, select_ws,
                     select_ws_bytes, stream=None):
    _check("vg_verify_select", lib().vg_verify_select(
        C.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(prefix_len), int(max_prefix),
        int(gamma), _ptr(out), _ptr(group_scores), _ptr(scores), _ptr(k), int(max_k), _ptr(sel_pos),
        _ptr(sel_slot), _ptr(sel_count), _ptr(verify_ws), int(verify_ws_bytes), _ptr(select_ws),
        int(select_ws_bytes), _stream(stream)))


def vg_sparse_draft_workspace_size(shape: VgShape, n_q: int, max_k: int, max_tail: int) -> int:
    n = C.c_size_t(0)
    _check("vg_sparse_draft_workspace_size", lib().vg_sparse_draft_workspace_size(
        C.byref(shape), int(n_q), int(max_k), int(max_tail), C.byref(n)))
    return n.value


def vg_sparse_draft_attention(shape, q, n_q, k_cache, v_cache, sel_slot, sel_count, max_k,
                              page_table, tail_start, tail_len, max_tail, out, workspace,
                              workspace_bytes, stream=None):
    _check("vg_sparse_draft_attention", lib().vg_sparse_draft_attention(
        C.byref(shape), _ptr(q), int(n_q), _ptr(k_cache), _ptr(v_cache), _ptr(sel_slot),
        _ptr(sel_count), int(max_k), _ptr(page_table), _ptr(tail_start), _ptr(tail_len),
        int(max_tail), _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def vg_sparse_draft_attention_noalloc(shape, q, n_q, k_cache, v_cache, sel_slot, sel_count, max_k,
                                      page_table, tail_start, tail_len, max_tail, out, stream=None):
    _check("vg_sparse_draft_attention_noalloc", lib().vg_sparse_draft_attention_noalloc(
        C.byref(shape), _ptr(q), int(n_q), _ptr(k_cache), _ptr(v_cache), _ptr(sel_slot),
        _ptr(sel_count), int(max_k), _ptr(page_table), _ptr(tail_start), _ptr(tail_len),
        int(max_tail), _ptr(out), _stream(stream)))


def vg_window_select(batch, max_prefix, prefix_len, k, max_k, n_sink, page_table, page_size, max_pages,
                     sel_pos, sel_slot, sel_count, stream=None):
    _check("vg_window_select", lib().vg_window_select(
        int(batch), int(max_prefix), _ptr(prefix_len), _ptr(k), int(max_k), int(n_sink), _ptr(page_table),
        int(page_size), int(max_pages), _ptr(sel_pos), _ptr(sel_slot), _ptr(sel_count), _stream(stream)))


def vg_kv_append(shape, k_new, v_new, n_new, page_table, start_pos, k_cache, v_cache, stream=None):
    _check("vg_kv_append", lib().vg_kv_append(
        C.byref(shape), _ptr(k_new), _ptr(v_new), int(n_new), _ptr(page_table), _ptr(start_pos),
        _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def vg_advance_prefix(batch, gamma, n_accepted, prefix_len, stream=None):
    _check("vg_advance_prefix", lib().vg_advance_prefix(
        int(batch), int(gamma), _ptr(n_accepted), _ptr(prefix_len), _stream(stream)))
