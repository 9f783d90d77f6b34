"""Parity gates shared by the GPU parity tests and the CPU test-power checks.

Each gate returns (ok, message).  The tolerances are the contract of the path:
  * page-table translation, gathered slots and index lists: bit-exact;
  * logits and scores: |x - x*| <= 1e-3 * (1 + |x*|);
  * attention outputs: |o - o*| <= 1e-2 absolute on unit-scale data;
  * top-k sets: equal, except positions whose oracle score lies within the
    score tolerance of the k-th oracle score.
The absolute output bound alone cannot tell a broken kernel from a correct
one when attention is nearly uniform over tens of thousands of keys (|o| is
then below 1e-2), so `output_gate` also applies a per-(sequence, row, head)
relative bound: max |o - o*| <= REL_OUT * RMS(o*) + 1e-6.  With bf16
probabilities in the P.V product the expected relative error is about
2^-9 / sqrt(3) ~ 1e-3 of the row's RMS, so REL_OUT = 5e-2 leaves a wide margin
while any wrong row, head map, mask or dropped key moves a row by O(RMS).
"""
from __future__ import annotations

import numpy as np

ABS_OUT = 1e-2
REL_OUT = 5e-2
SCORE_RTOL = 1e-3


def output_gate(o, o_ref, abs_tol=ABS_OUT, rel_tol=REL_OUT):
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    if o.shape != o_ref.shape:
        return False, f"shape {o.shape} != {o_ref.shape}"
    if not np.all(np.isfinite(o)):
        return False, "non-finite output"
    err = np.abs(o - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    if max_abs > abs_tol:
        return False, f"max abs error {max_abs:.3e} > {abs_tol}"
    blk_err = err.max(axis=-1)
    blk_rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1))
    ratio = blk_err / (rel_tol * blk_rms + 1e-6)
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        return False, (f"block {idx}: max err {float(blk_err[idx]):.3e} vs "
                       f"{rel_tol} x RMS {float(blk_rms[idx]):.3e}")
    return True, f"max abs {max_abs:.3e}, worst rel ratio {worst:.3f}"


def score_gate(x, x_ref, rtol=SCORE_RTOL, mask=None):
    """Elementwise |x - x*| <= rtol * (1 + |x*|) over `mask` (default: all)."""
    x = np.asarray(x, dtype=np.float64)
    x_ref = np.asarray(x_ref, dtype=np.float64)
    if x.shape != x_ref.shape:
        return False, f"shape {x.shape} != {x_ref.shape}"
    tol = rtol * (1.0 + np.abs(x_ref))
    bad = np.abs(x - x_ref) > tol
    if mask is not None:
        bad &= mask
    if np.any(~np.isfinite(x) & (mask if mask is not None else True)):
        return False, "non-finite values"
    n = int(bad.sum())
    if n:
        idx = np.unravel_index(int(np.argmax(bad)), bad.shape)
        return False, f"{n} entries out of tolerance, first at {idx}: {x[idx]} vs {x_ref[idx]}"
    err = np.abs(x - x_ref)
    if mask is not None:
        err = np.where(mask, err, 0.0)
    return True, f"max abs err {float(err.max()) if err.size else 0.0:.3e}"


def prefix_mask(prefix_len, max_prefix, lead_shape=()):
    """Boolean mask [B][*lead][max_prefix] true for j < P_b."""
    pl = np.asarray(prefix_len)
    m = np.arange(max_prefix)[None, :] < pl[:, None]
    for _ in lead_shape:
        m = m[:, None]
    return np.broadcast_to(m, (len(pl),) + tuple(lead_shape) + (max_prefix,))


def topk_gate(sel_pos, sel_count, scores_ref, prefix_len, k, rtol=SCORE_RTOL):
    """Per sequence: count == min(k, P); positions distinct, ascending, in [0, P);
    the set equals the oracle's top-k except for positions whose oracle score is
    within rtol * (1 + |s_k|) of the k-th largest oracle score."""
    sel_pos = np.asarray(sel_pos)
    for b in range(len(prefix_len)):
        P = int(prefix_len[b])
        kk = min(int(k[b]), P)
        c = int(sel_count[b])
        if c != kk:
            return False, f"seq {b}: count {c} != {kk}"
        if kk == 0:
            continue
        pos = sel_pos[b, :c].astype(np.int64)
        if np.any(pos < 0) or np.any(pos >= P):
            return False, f"seq {b}: position out of range"
        if np.any(np.diff(pos) <= 0):
            return False, f"seq {b}: positions not strictly ascending"
        s = np.asarray(scores_ref[b, :P], dtype=np.float64)
        kth = np.sort(s)[::-1][kk - 1]
        tol = rtol * (1.0 + abs(kth))
        chosen = np.zeros(P, dtype=bool)
        chosen[pos] = True
        must = s > kth + tol      # clearly above the threshold: must be chosen
        never = s < kth - tol     # clearly below: must not be chosen
        if np.any(must & ~chosen):
            return False, f"seq {b}: {int((must & ~chosen).sum())} clear top-k positions missing"
        if np.any(never & chosen):
            return False, f"seq {b}: {int((never & chosen).sum())} clearly-below positions chosen"
    return True, "ok"


def exact_gate(x, x_ref, what="values"):
    x = np.asarray(x)
    x_ref = np.asarray(x_ref)
    if x.shape != x_ref.shape:
        return False, f"{what}: shape {x.shape} != {x_ref.shape}"
    n = int(np.sum(x != x_ref))
    if n:
        idx = np.unravel_index(int(np.argmax(x != x_ref)), x.shape)
        return False, f"{what}: {n} mismatches, first at {idx}: {x[idx]} vs {x_ref[idx]}"
    return True, "bit-exact"
