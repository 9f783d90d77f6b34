"""Pins of the fp64 oracle against what the Vegas pages and mathematics fix.

None of these checks re-types the oracle's formulas: each compares it with a
brute-force enumeration, an independent library routine (torch's fp64
scaled_dot_product_attention, numpy's stable sort), a closed form, a
hand-derived worked example, or an invariant of the method.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from verification_guided_sparse_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return synth.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _logical(case, cache, b):
    """Dense logical [N_b][Hkv][D] float64 view of a paged cache (numpy gather)."""
    n = case.seq_len(b)
    pos = np.arange(n)
    slots = case.page_table[b, pos // case.page_size].astype(np.int64) * case.page_size + pos % case.page_size
    return _f64(cache)[slots]


def _tiny(dtype="bf16", prefix=(37,), gamma=3, hq=4, hkv=2, d=16, seed=7, paging="identity", **kw):
    cfg = synth.Config(name="tiny", batch=len(prefix), prefix=tuple(prefix), num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, dtype=dtype, gamma=gamma, k_pct=25,
                       sigma=1.0, hh_pct=10, sink=True, paging=paging, seed=seed, **kw)
    return synth.make_case(cfg)


# ---------------------------------------------------------------- selection

def _brute_best(scores, k):
    """All maximisers of sum_{i in T} s_i over |T| = k, by enumeration (lexicographic order)."""
    best, sets = None, []
    for T in itertools.combinations(range(len(scores)), k):
        v = sum(scores[i] for i in T)
        if best is None or v > best:
            best, sets = v, [T]
        elif v == best:
            sets.append(T)
    return best, sets


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("kind", ["distinct", "ties"])
def test_topk_is_subset_argmax(P, kind):
    """The selected set maximises the summed score over every size-k subset of
    the prefix (Vegas 2.A objective), for every k; with ties, the maximiser
    taking the lowest positions (lexicographically first) is the one returned."""
    rng = np.random.default_rng(100 + P)
    if kind == "distinct":
        s = rng.permutation(np.arange(P) - P // 2).astype(np.float64) / 1024.0 * 37.0
    else:
        s = rng.integers(-2, 3, size=P).astype(np.float64)  # many exact ties
    for k in range(0, P + 1):
        pos, _, cnt = oracle.topk(s[None], np.array([P]), np.array([k]), max_k=max(k, 1))
        assert cnt[0] == k
        T = tuple(int(x) for x in pos[0, :k])
        best, sets = _brute_best(list(s), k)
        assert T in sets, (k, T, best)
        if kind == "distinct":
            assert len(sets) == 1
        assert T == sets[0], "ties must go to the lowest positions"


def test_topk_clamps_and_matches_stable_sort():
    """k > P selects the whole prefix; larger cases match numpy's stable sort."""
    rng = np.random.default_rng(5)
    B, mp = 3, 500
    s = np.round(rng.standard_normal((B, mp)) * 64) / 64  # ties present
    P = np.array([500, 123, 7])
    k = np.array([50, 200, 3])
    pos, _, cnt = oracle.topk(s, P, k, max_k=200)
    for b in range(B):
        kk = min(k[b], P[b])
        assert cnt[b] == kk
        order = np.argsort(-s[b, :P[b]], kind="stable")[:kk]
        assert np.array_equal(pos[b, :kk], np.sort(order))
        # the same set as torch.topk where the k-th value is not tied
        vals = np.sort(s[b, :P[b]])[::-1]
        if kk < P[b] and vals[kk - 1] != vals[kk]:
            t = torch.topk(torch.from_numpy(s[b, :P[b]]), int(kk)).indices.numpy()
            assert np.array_equal(np.sort(t), pos[b, :kk])


def test_topk_slot_translation():
    case = _tiny(prefix=(40, 70), paging="permuted", gamma=2)
    rng = np.random.default_rng(1)
    s = rng.standard_normal((2, case.max_prefix))
    pos, slot, cnt = oracle.topk(s, case.prefix_len, case.k, page_table=case.page_table)
    for b in range(2):
        p = pos[b, :cnt[b]].astype(np.int64)
        expect = case.page_table[b, p // 16].astype(np.int64) * 16 + p % 16
        assert np.array_equal(slot[b, :cnt[b]], expect)


@pytest.mark.parametrize("shift", ["row_head_constant", "positive_scale"])
def test_selection_invariant_to_logit_normalisation(shift):
    """Adding a constant per (row, head) -- the log-softmax reading of 'logit' --
    or scaling all logits by c > 0 leaves the selected set unchanged."""
    rng = np.random.default_rng(9)
    B, Hq, mp = 2, 6, 300
    L = rng.integers(-4000, 4000, size=(B, 2, Hq, mp)).astype(np.float64) / 1024.0
    P = np.array([300, 211])
    k = np.array([30, 17])
    base = oracle.topk(oracle.aggregate(L, P), P, k)[0]
    if shift == "row_head_constant":
        c = rng.integers(-5000, 5000, size=(B, 2, Hq, 1)).astype(np.float64) / 1024.0
        L2 = L + c
        got = oracle.topk(oracle.aggregate(L2, P), P, k)[0]
        assert np.array_equal(base, got)
    else:
        for c in (0.25, 3.0, 64.0):
            got = oracle.topk(oracle.aggregate(L * c, P), P, k)[0]
            assert np.array_equal(base, got)


def test_aggregate_against_numpy_sum():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((2, 2, 8, 50))
    P = np.array([50, 20])
    s = oracle.aggregate(L, P)
    ref = L.sum(axis=(1, 2))
    assert np.allclose(s[0], ref[0], rtol=0, atol=1e-12)
    assert np.allclose(s[1, :20], ref[1, :20], rtol=0, atol=1e-12)
    assert np.all(s[1, 20:] == 0)


# ---------------------------------------------------------------- attention

def _sdpa_ref(case, rows_q, visible):
    """torch fp64 scaled_dot_product_attention over the dense logical cache.
    visible(b, r) -> number of leading logical keys row r may see."""
    outs = []
    G = case.num_q_heads // case.num_kv_heads
    for b in range(case.batch):
        K = torch.from_numpy(_logical(case, case.k_cache, b)).permute(1, 0, 2)  # [Hkv][N][D]
        V = torch.from_numpy(_logical(case, case.v_cache, b)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).unsqueeze(0)
        V = V.repeat_interleave(G, dim=0).unsqueeze(0)
        q = torch.from_numpy(_f64(rows_q[b])).permute(1, 0, 2).unsqueeze(0)  # [1][Hq][R][D]
        R, N = q.shape[2], K.shape[2]
        mask = torch.zeros(R, N, dtype=torch.bool)
        for r in range(R):
            mask[r, : visible(b, r)] = True
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=case.scale)
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.stack(outs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("paging", ["identity", "permuted"])
def test_verify_matches_torch_sdpa(dtype, paging):
    case = _tiny(dtype=dtype, prefix=(61, 33), gamma=4, hq=8, hkv=2, d=32, paging=paging)
    out, logits, group, lall = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table,
                                             case.prefix_len, case.gamma, case.scale, export="all")
    ref = _sdpa_ref(case, case.q, lambda b, r: int(case.prefix_len[b]) + r + 1)
    assert np.max(np.abs(out - ref)) < 1e-10
    # exported logits = scale * q.k of rows 0 and gamma, independent einsum
    G = case.num_q_heads // case.num_kv_heads
    for b in range(case.batch):
        P = int(case.prefix_len[b])
        K = _logical(case, case.k_cache, b)[:P]  # [P][Hkv][D]
        Kh = np.repeat(K, G, axis=1)  # [P][Hq][D]
        q = _f64(case.q[b])  # [R][Hq][D]
        l = np.einsum("rhd,jhd->rhj", q, Kh) * case.scale
        assert np.max(np.abs(logits[b, 0, :, :P] - l[0])) < 1e-12
        assert np.max(np.abs(logits[b, 1, :, :P] - l[case.gamma])) < 1e-12
        assert np.max(np.abs(lall[b, :, :, :P] - l)) < 1e-12
        assert np.all(logits[b, :, :, P:] == 0)
        gsum = (l[0] + l[case.gamma]).reshape(case.num_kv_heads, G, P).sum(axis=1)
        assert np.max(np.abs(group[b, :, :P] - gsum)) < 1e-12


def test_softmax_weights_via_one_hot_values():
    """With V[j] = e_j (one-hot), the output row is the probability vector: it is
    non-negative, sums to 1, matches numpy's softmax of the scaled scores, and is
    exactly 0 on the causally masked positions."""
    P, gamma, D, Hq, Hkv = 9, 3, 16, 4, 2
    case = _tiny(dtype="f32", prefix=(P,), gamma=gamma, hq=Hq, hkv=Hkv, d=D)
    N = P + gamma + 1
    v = np.zeros_like(case.v_cache)
    pos = np.arange(N)
    slots = case.page_table[0, pos // 16] * 16 + pos % 16
    for j in range(N):
        v[slots[j], :, j] = 1.0
    out = oracle.verify(case.q, case.k_cache, v, case.page_table, case.prefix_len, gamma, case.scale)[0]
    K = _logical(case, case.k_cache, 0)
    G = Hq // Hkv
    for r in range(gamma + 1):
        for h in range(Hq):
            p = out[0, r, h]
            vis = P + r + 1
            l = K[:vis, h // G] @ _f64(case.q[0, r, h]) * case.scale
            e = np.exp(l - l.max())
            assert np.all(p >= 0)
            assert abs(p.sum() - 1.0) < 1e-12
            assert np.max(np.abs(p[:vis] - e / e.sum())) < 1e-13
            assert np.all(p[vis:] == 0.0)


def test_causal_mask_perturbation():
    """Changing K/V after position P + r leaves row r bit-identical; changing a
    visible position changes it."""
    case = _tiny(dtype="bf16", prefix=(50,), gamma=4)
    base = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table, case.prefix_len, 4, case.scale)[0]
    P = 50
    for j in range(P + 1, P + 5):
        k2 = case.k_cache.copy()
        v2 = case.v_cache.copy()
        s = case.page_table[0, j // 16] * 16 + j % 16
        k2[s] ^= np.uint16(0x0100)
        v2[s] ^= np.uint16(0x0100)
        o2 = oracle.verify(case.q, k2, v2, case.page_table, case.prefix_len, 4, case.scale)[0]
        for r in range(5):
            if P + r < j:
                assert np.array_equal(o2[0, r], base[0, r]), (j, r)
            else:
                assert not np.array_equal(o2[0, r], base[0, r]), (j, r)


def test_page_permutation_invariance():
    """Identical logical data under a permuted page table gives bit-identical results."""
    a = _tiny(prefix=(77, 40), paging="identity", gamma=3)
    b = _tiny(prefix=(77, 40), paging="permuted", gamma=3)
    assert not np.array_equal(a.page_table, b.page_table)
    ra = oracle.verify(a.q, a.k_cache, a.v_cache, a.page_table, a.prefix_len, 3, a.scale)
    rb = oracle.verify(b.q, b.k_cache, b.v_cache, b.page_table, b.prefix_len, 3, b.scale)
    for x, y in zip(ra[:3], rb[:3]):
        assert np.array_equal(x, y)


def test_thread_count_does_not_change_results():
    """The oracle's thread units (one per sequence and query head, then one per
    sequence and KV head for the group export) each compute a fixed set of
    outputs in a fixed order: one thread and many give bit-identical results."""
    c = _tiny(prefix=(77, 40), gamma=3, hq=8, hkv=2)
    one = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len, 3, c.scale, nthreads=1)
    many = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len, 3, c.scale, nthreads=7)
    for x, y in zip(one[:3], many[:3]):
        assert np.array_equal(x, y)
    s = oracle.aggregate(one[2], c.prefix_len)
    pos, _, cnt = oracle.topk(s, c.prefix_len, np.array([9, 5]), page_table=c.page_table)
    args = (np.ascontiguousarray(c.q_draft[1][:, None]), c.k_cache, c.v_cache, c.page_table, pos, cnt,
            c.prefix_len, np.array([2, 2], np.int32), c.scale)
    assert np.array_equal(oracle.sparse(*args, nthreads=1), oracle.sparse(*args, nthreads=5))


def test_closed_forms():
    case = _tiny(dtype="f32", prefix=(20,), gamma=2, hq=2, hkv=1, d=8)
    # all keys equal -> uniform weights -> mean of the visible values
    k_eq = np.broadcast_to(case.k_cache[:1], case.k_cache.shape).copy()
    out = oracle.verify(case.q, k_eq, case.v_cache, case.page_table, case.prefix_len, 2, case.scale)[0]
    V = _logical(case, case.v_cache, 0)
    for r in range(3):
        assert np.max(np.abs(out[0, r] - V[: 20 + r + 1, 0].mean(axis=0))) < 1e-13
    # q = 0 -> uniform weights as well
    out0 = oracle.verify(np.zeros_like(case.q), case.k_cache, case.v_cache, case.page_table,
                         case.prefix_len, 2, case.scale)[0]
    for r in range(3):
        assert np.max(np.abs(out0[0, r] - V[: 20 + r + 1, 0].mean(axis=0))) < 1e-13
    # one visible key (empty prefix, row 0) -> exactly that value row
    out1 = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table, np.array([0]), 2,
                         case.scale, max_prefix=0)[0]
    assert np.array_equal(out1[0, 0], np.repeat(V[0:1, 0], 2, axis=0))
    # sparse with nothing selected and a one-token tail -> exactly that value row
    o = oracle.sparse(case.q[:, :1], case.k_cache, case.v_cache, case.page_table,
                      np.zeros((1, 1), np.int32), np.array([0]), np.array([5]), np.array([1]), case.scale)
    assert np.array_equal(o[0, 0], np.repeat(V[5:6, 0], 2, axis=0))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sparse_over_whole_prefix_equals_verify(dtype):
    """Selecting every prefix position (k = P) and the tail [P, P + r] reproduces
    verify row r: page-size-1 sparse attention is attention over its index list."""
    case = _tiny(dtype=dtype, prefix=(45, 30), gamma=3, hq=4, hkv=2, d=16)
    out = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table, case.prefix_len, 3, case.scale)[0]
    mk = case.max_prefix
    sel = np.full((2, mk), -1, np.int32)
    for b in range(2):
        sel[b, : case.prefix_len[b]] = np.arange(case.prefix_len[b])
    for r in range(4):
        o = oracle.sparse(np.ascontiguousarray(case.q[:, r:r + 1]), case.k_cache, case.v_cache,
                          case.page_table, sel, case.prefix_len, case.prefix_len,
                          np.array([r + 1, r + 1]), case.scale)
        assert np.max(np.abs(o[:, 0] - out[:, r])) < 1e-12


def test_sparse_matches_torch_over_index_list():
    """Sparse draft = softmax attention over exactly sel ++ causal tail (torch fp64)."""
    case = _tiny(dtype="bf16", prefix=(90,), gamma=4, hq=4, hkv=2, d=16, paging="permuted")
    rng = np.random.default_rng(4)
    sel = np.sort(rng.choice(90, size=12, replace=False)).astype(np.int32)[None]
    n_q, tail_len = 2, 4
    q = np.ascontiguousarray(case.q[:, :n_q])
    o = oracle.sparse(q, case.k_cache, case.v_cache, case.page_table, sel, np.array([12]),
                      np.array([90]), np.array([tail_len]), case.scale)
    K = _logical(case, case.k_cache, 0)
    V = _logical(case, case.v_cache, 0)
    G = 2
    for row in range(n_q):
        idx = list(sel[0]) + list(range(90, 90 + tail_len - n_q + row + 1))
        for h in range(4):
            qq = torch.from_numpy(_f64(q[0, row, h]))[None, None, None]
            kk = torch.from_numpy(K[idx, h // G])[None, None]
            vv = torch.from_numpy(V[idx, h // G])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=case.scale)
            assert np.max(np.abs(o[0, row, h] - ref[0, 0, 0].numpy())) < 1e-12


def test_handworked_example():
    """A 3-key example worked out by hand (tests/golden/handworked_3key.json)."""
    with open(os.path.join(GOLDEN, "handworked_3key.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float32).reshape(1, 1, 1, 2)
    kc = np.zeros((16, 1, 2), np.float32)
    vc = np.zeros((16, 1, 2), np.float32)
    kc[:3, 0] = np.array(g["k"], dtype=np.float32)
    vc[:3, 0] = np.array(g["v"], dtype=np.float32)
    pt = np.zeros((1, 1), np.int32)
    out, logits, _, _ = oracle.verify(q, kc, vc, pt, np.array([2]), 0, g["scale"])
    assert np.max(np.abs(out[0, 0, 0] - np.array(g["out"]))) < 1e-6
    assert np.max(np.abs(logits[0, 0, 0] - np.array(g["logits_row0"], dtype=np.float32))) < 1e-7
    s = oracle.aggregate(logits, np.array([2]))
    assert np.max(np.abs(s[0] - np.array(g["scores"]))) < 1e-6
    pos, _, _ = oracle.topk(s, np.array([2]), np.array([1]))
    assert pos[0, 0] == g["top1"]


def test_k_rule_reproduces_workload_sizes():
    """k = round-half-up(pct% of P) reproduces the selection sizes of the five workloads."""
    got = {n: int(synth.pct_round_half_up(c.prefix[0] if c.prefix else 0, c.k_pct))
           for n, c in synth.CONFIGS.items() if c.prefix}
    assert got == {"c1_tiny": 205, "c2_qwen3_32k": 1638, "c3_qwen3_128k": 5243, "c5_gptoss_64k": 3277}
    assert math.floor(2048 * 0.02 + 0.5) == synth.pct_round_half_up(2048, 2) == 41


def test_full_collection_scores_are_the_literal_objective():
    """Full collection: every verify row exported; the aggregated score of position j
    is the per-position coefficient of the section 2.A objective summed over all
    gamma+1 rows and all heads (independent einsum), and the group form summed over
    KV heads gives the same scores."""
    case = _tiny(prefix=(23, 9), gamma=3, hq=8, hkv=2, d=16)
    _, logits, group, lall = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table,
                                           case.prefix_len, case.gamma, case.scale, export="all")
    s_all = oracle.aggregate(lall, case.prefix_len)
    s_grp = oracle.aggregate(oracle.group_sums(lall, case.num_kv_heads), case.prefix_len)
    G = case.num_q_heads // case.num_kv_heads
    for b in range(case.batch):
        P = int(case.prefix_len[b])
        K = np.repeat(_logical(case, case.k_cache, b)[:P], G, axis=1)
        coef = np.einsum("rhd,jhd->j", _f64(case.q[b]), K) * case.scale  # sum over rows and heads
        assert np.max(np.abs(s_all[b, :P] - coef)) < 1e-10
        assert np.max(np.abs(s_grp[b, :P] - coef)) < 1e-10
        assert np.all(s_all[b, P:] == 0)


def test_group_sums_match_the_c_export():
    """oracle.group_sums over the two exported rows equals the C oracle's own group export."""
    case = _tiny(prefix=(40, 17), gamma=4, hq=8, hkv=4, d=16)
    _, logits, group, _ = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table,
                                        case.prefix_len, case.gamma, case.scale)
    assert np.max(np.abs(oracle.group_sums(logits, case.num_kv_heads) - group)) < 1e-12


def test_two_row_collection_is_full_at_gamma_one():
    """With gamma = 1 the first draft row and the bonus row are all the rows."""
    case = _tiny(prefix=(30,), gamma=1, hq=4, hkv=2, d=16)
    _, logits, group, lall = oracle.verify(case.q, case.k_cache, case.v_cache, case.page_table,
                                           case.prefix_len, case.gamma, case.scale, export="all")
    assert np.array_equal(logits, lall)
    assert np.max(np.abs(oracle.group_sums(lall, case.num_kv_heads) - group)) < 1e-12


def test_kv_append_rebuilds_the_cache():
    """Writing each sequence's new tokens (read back through the page table) into a
    cache whose new-token slots were cleared reproduces the cache exactly."""
    case = _tiny(prefix=(37, 5, 20), gamma=3, hq=4, hkv=2, d=16, paging="permuted")
    R = case.rows

    def raw_rows(cache, b):  # the stored rows (raw bits) of positions P_b .. P_b + gamma
        pos = np.arange(int(case.prefix_len[b]), int(case.prefix_len[b]) + R)
        return cache[case.page_table[b, pos // 16].astype(np.int64) * 16 + pos % 16]

    k_new = np.stack([raw_rows(case.k_cache, b) for b in range(case.batch)])
    v_new = np.stack([raw_rows(case.v_cache, b) for b in range(case.batch)])
    k0, v0 = case.k_cache.copy(), case.v_cache.copy()
    for b in range(case.batch):
        for r in range(R):
            p = int(case.prefix_len[b]) + r
            slot = int(case.page_table[b][p // 16]) * 16 + p % 16
            k0[slot] = 0
            v0[slot] = 0
    assert not np.array_equal(k0, case.k_cache)
    k1, v1 = oracle.kv_append(k0, v0, k_new, v_new, case.page_table, case.prefix_len)
    assert np.array_equal(k1, case.k_cache) and np.array_equal(v1, case.v_cache)


def test_iterations_grow_the_logical_sequence():
    """Append the new tokens, keep the first and the accepted drafts, repeat: each
    sequence read back in position order through its page table is the starting
    prefix followed, per iteration, by the first new token and the accepted drafts
    (the rejected drafts' slots are overwritten by the next append)."""
    case = _tiny(prefix=(37, 21, 30), gamma=3, hq=4, hkv=2, d=16, paging="permuted")
    R, n_iter = case.rows, 2
    p = (case.prefix_len - n_iter * R).astype(np.int32)  # the pages cover prefix_len + R
    assert (p > 0).all()
    k, v = case.k_cache.copy(), case.v_cache.copy()

    def logical(cache, b, n):
        pos = np.arange(n)
        return cache[case.page_table[b, pos // 16].astype(np.int64) * 16 + pos % 16]

    want_k = [list(logical(k, b, int(p[b]))) for b in range(case.batch)]
    want_v = [list(logical(v, b, int(p[b]))) for b in range(case.batch)]
    for it in range(n_iter):
        k_new, v_new = synth.new_token_rows(case, it)
        k, v = oracle.kv_append(k, v, k_new, v_new, case.page_table, p)
        n = synth.accepted_counts(case, it)
        assert ((n >= 0) & (n <= case.gamma)).all()
        p = oracle.advance_prefix(p, n, case.gamma)
        for b in range(case.batch):
            want_k[b] += list(k_new[b, : 1 + n[b]])
            want_v[b] += list(v_new[b, : 1 + n[b]])
    for b in range(case.batch):
        assert len(want_k[b]) == p[b]
        assert np.array_equal(logical(k, b, int(p[b])), np.stack(want_k[b]))
        assert np.array_equal(logical(v, b, int(p[b])), np.stack(want_v[b]))
    # counts outside [0, gamma] are clamped; writes past the page-table row are skipped
    assert list(oracle.advance_prefix([10, 10, 10], [-3, 2, 99], 3)) == [11, 13, 14]
    far = np.full(case.batch, case.page_table.shape[1] * 16, np.int32)
    k2, _ = oracle.kv_append(k, v, k_new, v_new, case.page_table, far)
    assert np.array_equal(k2, k)


@pytest.mark.parametrize("n_sink", [0, 1, 4, 16])
def test_window_select_is_topk_of_a_recency_score(n_sink):
    """The query-agnostic selection equals the exact top-k of a score that ranks
    the sink positions above everything and the rest by recency (a special case
    of the pinned top-k): same positions and slots, for k from 0 past P."""
    case = _tiny(prefix=(37, 5, 20, 1), gamma=2, paging="permuted")
    P = case.prefix_len
    mp = int(P.max())
    j = np.arange(mp, dtype=np.float64)
    score = np.where(j < n_sink, 1e6, j)[None].repeat(len(P), 0)
    for kv in (0, 1, 3, 4, 5, 17, 40):
        k = np.full(len(P), kv, np.int32)
        pos, slot, cnt = oracle.window_select(P, k, n_sink, case.page_table, max_k=max(kv, 1))
        tp, ts, tc = oracle.topk(score, P, k, page_table=case.page_table, max_k=max(kv, 1))
        assert np.array_equal(cnt, tc)
        for b in range(len(P)):
            n = int(cnt[b])
            assert np.array_equal(pos[b, :n], tp[b, :n]) and np.array_equal(slot[b, :n], ts[b, :n]), (kv, b)
