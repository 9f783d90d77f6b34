"""Test power of the parity gates, checked on the CPU.

Each case plants a plausible kernel mistake in the oracle's own result (never
on the GPU) and asserts that the gates the GPU parity tests use reject it,
while the oracle's correct result passes them.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import parity
from verification_guided_sparse_amd import synth


def _case(sharp):
    cfg = synth.small("c1_tiny", prefix=(2048,))
    if sharp:
        cfg = synth.sharp(cfg)
    return synth.make_case(cfg)


@pytest.fixture(scope="module", params=[False, True], ids=["c1", "c1_sharp"])
def ref(request):
    c = _case(request.param)
    out, logits, group, lall = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len,
                                             c.gamma, c.scale, export="all")
    return c, out, logits, lall


def _sparse_rows(c, sel_lists, extra_tail):
    """Row r of the verify output recomputed over [sel] ++ [P, P + r + extra_tail]."""
    P = int(c.prefix_len[0])
    out = np.zeros((1, c.rows, c.num_q_heads, c.head_dim))
    for r in range(c.rows):
        sel = np.asarray(sel_lists, dtype=np.int32)[None]
        tl = min(r + 1 + extra_tail, c.rows)
        out[:, r] = oracle.sparse(np.ascontiguousarray(c.q[:, r:r + 1]), c.k_cache, c.v_cache,
                                  c.page_table, sel, np.array([sel.shape[1]]), np.array([P]),
                                  np.array([tl]), c.scale)[:, 0]
    return out


def test_correct_result_passes(ref):
    c, out, logits, _ = ref
    assert parity.output_gate(out, out)[0]
    assert parity.score_gate(logits, logits)[0]


def test_zero_output_rejected(ref):
    c, out, _, _ = ref
    assert not parity.output_gate(np.zeros_like(out), out)[0]


def test_wrong_gqa_map_rejected(ref):
    """Kernel reads KV head h % Hkv instead of h // G."""
    c, out, _, _ = ref
    Hq, Hkv = c.num_q_heads, c.num_kv_heads
    G = Hq // Hkv
    perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
    q2 = np.empty_like(c.q)
    q2[:, :, perm] = c.q
    o2 = oracle.verify(q2, c.k_cache, c.v_cache, c.page_table, c.prefix_len, c.gamma, c.scale)[0]
    wrong = o2[:, :, perm]
    assert not parity.output_gate(wrong, out)[0]


@pytest.mark.parametrize("sharp", [False, True])
def test_causal_off_by_one_rejected(sharp):
    """Row r sees one key too many (P + r + 1).  One extra key among thousands can
    hide in a long row, so the parity suite runs short prefixes where it cannot;
    here: P = 40."""
    cfg = synth.small("c1_tiny", prefix=(40,))
    c = synth.make_case(synth.sharp(cfg) if sharp else cfg)
    out = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len, c.gamma, c.scale)[0]
    wrong = _sparse_rows(c, np.arange(40), extra_tail=1)
    assert not parity.output_gate(wrong, out)[0]


def test_dropped_page_rejected(ref):
    """One 16-token page of the prefix is skipped: the output or the exported logits must fail."""
    c, out, logits, _ = ref
    P = int(c.prefix_len[0])
    keep = np.setdiff1d(np.arange(P), np.arange(16 * 37, 16 * 38))
    wrong = _sparse_rows(c, keep, extra_tail=0)
    wrong_logits = logits.copy()
    wrong_logits[..., 16 * 37: 16 * 38] = 0.0
    assert not (parity.output_gate(wrong, out)[0] and parity.score_gate(wrong_logits, logits)[0])
    assert not parity.score_gate(wrong_logits, logits)[0]


def test_wrong_export_row_rejected(ref):
    """Row gamma-1 exported instead of the bonus row gamma."""
    c, _, logits, lall = ref
    wrong = logits.copy()
    wrong[:, 1] = lall[:, c.gamma - 1]
    assert not parity.score_gate(wrong, logits)[0]


def test_score_missing_head_rejected(ref):
    c, _, logits, _ = ref
    s = oracle.aggregate(logits, c.prefix_len)
    l2 = logits.copy()
    l2[:, :, 3] = 0.0
    s_wrong = oracle.aggregate(l2, c.prefix_len)
    assert parity.score_gate(s, s)[0]
    assert not parity.score_gate(s_wrong, s)[0]


def test_topk_mistakes_rejected(ref):
    c, _, logits, _ = ref
    s = oracle.aggregate(logits, c.prefix_len)
    pos, _, cnt = oracle.topk(s, c.prefix_len, c.k)
    assert parity.topk_gate(pos, cnt, s, c.prefix_len, c.k)[0]
    # one element short
    assert not parity.topk_gate(pos[:, :-1], cnt - 1, s, c.prefix_len, c.k)[0]
    # the smallest selected swapped for the best unselected-but-clearly-lower one
    bad = pos.copy()
    P = int(c.prefix_len[0])
    order = np.argsort(-s[0, :P], kind="stable")
    bad[0, np.argmin(s[0, pos[0]])] = order[int(c.k[0]) + 20]
    bad[0] = np.sort(bad[0])
    assert not parity.topk_gate(bad, cnt, s, c.prefix_len, c.k)[0]
    # descending order is not the contract
    assert not parity.topk_gate(pos[:, ::-1], cnt, s, c.prefix_len, c.k)[0]
