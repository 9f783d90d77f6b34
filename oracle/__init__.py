"""fp64 CPU oracle for one decode iteration of Vegas's verification-guided sparse attention.

TEST INFRASTRUCTURE.  Only tests, the package smoke check and the benchmark's
CPU-baseline leg may import this package.  It is plain C (vegas_oracle.c,
built by oracle/build.py with gcc) behind a ctypes wrapper that only
marshals numpy arrays; it shares no code with the HIP library.

Functions take the host arrays produced by the seeded generator (bf16 as
uint16 bit patterns, or float32) and return float64 / int32 numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(path)
        P = C.c_void_p
        i32 = C.c_int
        L.oracle_verify.argtypes = [i32] * 7 + [C.c_double] + [P] * 5 + [i32, i32] + [P] * 4 + [i32]
        L.oracle_aggregate.argtypes = [i32, i32, i32, i32, P, P, P]
        L.oracle_topk.argtypes = [i32, i32, P, P, P, i32, P, i32, i32, P, P, P]
        L.oracle_sparse.argtypes = ([i32] * 7 + [C.c_double, P, i32, P, P, P, P, P, i32, P, P, P, i32])
        for f in (L.oracle_verify, L.oracle_aggregate, L.oracle_topk, L.oracle_sparse):
            f.restype = i32
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _dt(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return 1
    if x.dtype == np.float32:
        return 0
    raise TypeError("inputs must be bf16 bits (uint16) or float32")


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def verify(q, k_cache, v_cache, page_table, prefix_len, gamma, scale, *, page_size=16,
           max_prefix=None, export="two", nthreads=0):
    """Full causal verify attention with the Collect-2-Query export.

    Returns (out [B][R][Hq][D], logits [B][2][Hq][max_prefix],
    group [B][Hkv][max_prefix], logits_all or None).  `export="all"` also
    returns every row's logits [B][R][Hq][max_prefix] (full collection).
    Export entries j >= P_b are zero.
    """
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    B, R, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    assert R == gamma + 1 and k_cache.shape[2] == D and v_cache.shape == k_cache.shape
    pt = _c(page_table, np.int32)
    pl = _c(prefix_len, np.int32)
    mp = int(pl.max()) if max_prefix is None else int(max_prefix)
    out = np.zeros((B, R, Hq, D), dtype=np.float64)
    logits = np.zeros((B, 2, Hq, mp), dtype=np.float64)
    group = np.zeros((B, Hkv, mp), dtype=np.float64)
    lall = np.zeros((B, R, Hq, mp), dtype=np.float64) if export == "all" else None
    rc = lib().oracle_verify(B, Hq, Hkv, D, page_size, pt.shape[1], _dt(q), float(scale), _p(q),
                             _p(k_cache), _p(v_cache), _p(pt), _p(pl), int(gamma), mp, _p(out),
                             _p(logits), _p(group), _p(lall), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_verify failed ({rc})")
    return out, logits, group, lall


def kv_append(k_cache, v_cache, k_new, v_new, page_table, start_pos, page_size=16):
    """Copies of the caches with the new tokens' rows written at their slots:
    cache[page_table[b][p // ps] * ps + p % ps] = new[b][r] for p = start_pos[b] + r
    (the append that precedes verification: verify attends to the gamma + 1 new
    tokens from the cache, Vegas section 2, core mechanism).  Positions whose
    page-table entry lies outside the row or is negative are skipped."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    B, n_new = k_new.shape[:2]
    max_pages = page_table.shape[1]
    for b in range(B):
        for r in range(n_new):
            p = int(start_pos[b]) + r
            if p < 0 or p // page_size >= max_pages or page_table[b][p // page_size] < 0:
                continue
            slot = int(page_table[b][p // page_size]) * page_size + p % page_size
            k[slot] = k_new[b, r]
            v[slot] = v_new[b, r]
    return k, v


def window_select(prefix_len, k, n_sink, page_table=None, page_size=16, max_k=None):
    """Query-agnostic selection (the sliding-window style baseline of Vegas
    section 1): the first min(n_sink, kk) prefix positions and the most recent
    ones, kk = min(k_b, P_b) in all, ascending; with their page-size-1 slots.
    Returns (pos [B][max_k], slot [B][max_k], count [B]), unwritten entries -1."""
    B = len(prefix_len)
    mk = max(1, int(max(k)) if max_k is None else int(max_k))
    pos = np.full((B, mk), -1, dtype=np.int32)
    slot = np.full((B, mk), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        P = int(prefix_len[b])
        kk = min(int(k[b]), P, mk)
        chosen = sorted(set(range(min(n_sink, kk))) | set(range(P - (kk - min(n_sink, kk)), P)))
        assert len(chosen) == kk
        for i, j in enumerate(chosen):
            pos[b, i] = j
            if page_table is not None:
                slot[b, i] = int(page_table[b][j // page_size]) * page_size + j % page_size
        cnt[b] = kk
    return pos, slot, cnt


def advance_prefix(prefix_len, n_accepted, gamma):
    """Prefix lengths after an iteration: the sequence keeps its first new token
    and the n accepted drafts (clamped to [0, gamma]) of the gamma + 1 tokens
    verification judged (Vegas section 2, core mechanism)."""
    return np.array([int(p) + 1 + min(max(int(n), 0), int(gamma)) for p, n in zip(prefix_len, n_accepted)],
                    dtype=np.int32)


def group_sums(src, num_kv_heads):
    """Group form of an export [B][T][Hq][max_prefix]: the sum over its T rows and
    the G = Hq / Hkv consecutive query heads of each KV head -> [B][Hkv][max_prefix]
    (the per-KV-head part of the selection objective, Vegas section 2.A)."""
    src = np.asarray(src, dtype=np.float64)
    B, T, Hq, mp = src.shape
    G = Hq // int(num_kv_heads)
    return src.reshape(B, T, int(num_kv_heads), G, mp).sum(axis=(1, 3))


def aggregate(src, prefix_len, max_prefix=None):
    """Scores s[b][j] = sum over rows t and heads h of src[b][t][h][j], j < P_b (else 0).

    `src` is [B][T][Hq][max_prefix] (T = 2 for Collect-2-Query, gamma+1 for full
    collection) or the group form [B][Hkv][max_prefix] (summed over its heads).
    """
    src = _c(src, np.float64)
    if src.ndim == 3:
        src = src[:, None]
    B, T, H, mp = src.shape
    pl = _c(prefix_len, np.int32)
    scores = np.zeros((B, mp), dtype=np.float64)
    rc = lib().oracle_aggregate(B, H, T, mp, _p(pl), _p(src), _p(scores))
    if rc != 0:
        raise ValueError(f"oracle_aggregate failed ({rc})")
    return scores


def topk(scores, prefix_len, k, page_table=None, page_size=16, max_k=None):
    """Exact top-k per sequence: returns (sel_pos [B][max_k], sel_slot or None, sel_count [B]).

    Positions are ascending; ties at the k-th score go to the lower positions;
    unused entries are -1.
    """
    scores = _c(scores, np.float64)
    B, mp = scores.shape
    pl = _c(prefix_len, np.int32)
    kk = _c(k, np.int32)
    mk = int(kk.max()) if max_k is None else int(max_k)
    sel_pos = np.full((B, max(mk, 1)), -1, dtype=np.int32)
    sel_slot = np.full((B, max(mk, 1)), -1, dtype=np.int32) if page_table is not None else None
    cnt = np.zeros(B, dtype=np.int32)
    pt = _c(page_table, np.int32) if page_table is not None else None
    rc = lib().oracle_topk(B, mp, _p(scores), _p(pl), _p(kk), mk, _p(pt), int(page_size),
                           int(pt.shape[1]) if pt is not None else 0, _p(sel_pos), _p(sel_slot),
                           _p(cnt))
    if rc != 0:
        raise ValueError(f"oracle_topk failed ({rc})")
    return sel_pos[:, :mk], (sel_slot[:, :mk] if sel_slot is not None else None), cnt


def sparse(q, k_cache, v_cache, page_table, sel_pos, sel_count, tail_start, tail_len, scale, *,
           page_size=16, nthreads=0):
    """Sparse draft attention over the selected positions plus the causal tail.

    q [B][n_q][Hq][D]; sel_pos [B][max_k] logical positions.  Returns out [B][n_q][Hq][D].
    """
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    B, nq, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    pt = _c(page_table, np.int32)
    sp = _c(sel_pos, np.int32)
    if sp.ndim == 1:
        sp = sp[None]
    mk = sp.shape[1]
    cnt = _c(sel_count, np.int32)
    ts = _c(tail_start, np.int32)
    tl = _c(tail_len, np.int32)
    out = np.zeros((B, nq, Hq, D), dtype=np.float64)
    rc = lib().oracle_sparse(B, Hq, Hkv, D, page_size, pt.shape[1], _dt(q), float(scale), _p(q),
                             nq, _p(k_cache), _p(v_cache), _p(pt), _p(sp) if mk else None,
                             _p(cnt), mk, _p(ts), _p(tl), _p(out), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_sparse failed ({rc})")
    return out
