"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Each step is checked in isolation on the oracle's own inputs (fp32-rounded
where the GPU step consumes fp32), then the chain end to end.  Gates are the
contract tolerances of tests/parity.py; integer outputs are bit-exact.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

import oracle
from tests import parity
from verification_guided_sparse_amd import synth

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    from verification_guided_sparse_amd import _binding
    _binding.lib()  # fail loudly if the HIP library is missing
    return torch


def _oracle_all(c):
    out, logits, group, _ = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len,
                                          c.gamma, c.scale, nthreads=NTHREADS)
    return out, logits, group


def _rows_mask(c, lead):
    return parity.prefix_mask(c.prefix_len, c.max_prefix, lead)


def _check(ok_msg, what):
    ok, msg = ok_msg
    assert ok, f"{what}: {msg}"


def _run_steps(c, kernel=None, pad=64):
    """Per-step parity of one case; returns the device case for further checks."""
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd.runner import DeviceCase
    import torch
    _say(f"[parity] {c.cfg.name} B={c.batch} P={list(c.prefix_len)} Hq={c.num_q_heads} "
         f"Hkv={c.num_kv_heads} D={c.head_dim} {c.dtype} gamma={c.gamma} kernel={kernel} pad={pad}")
    dc = DeviceCase(c, kernel=vg.VG_KERNEL_AUTO if kernel is None else kernel, pad=pad)
    out_ref, logits_ref, group_ref = _oracle_all(c)

    # verify + export (both forms)
    dc.verify(export="both")
    torch.cuda.synchronize()
    _check(parity.output_gate(dc.host("out"), out_ref), "verify out")
    _check(parity.score_gate(dc.host("logits"), logits_ref, mask=_rows_mask(c, (2, c.num_q_heads))),
           "verify logits")
    _check(parity.score_gate(dc.host("group"), group_ref, mask=_rows_mask(c, (c.num_kv_heads,))),
           "verify group scores")

    # aggregate on the oracle's logits (fp32-rounded), both sources
    dc.put("logits", logits_ref.astype(np.float32))
    dc.put("group", group_ref.astype(np.float32))
    mask_s = _rows_mask(c, ())
    for src, ref_src in (("raw", logits_ref.astype(np.float32)), ("group", group_ref.astype(np.float32))):
        dc.aggregate(src=src)
        torch.cuda.synchronize()
        s_ref = oracle.aggregate(ref_src.astype(np.float64), c.prefix_len)
        _check(parity.score_gate(dc.host("scores"), s_ref, mask=mask_s), f"aggregate {src}")

    # aggregation + top-k in one call on the oracle's exports: scores within
    # the score tolerance, and the selection bit-exact against the oracle's
    # top-k of the GPU's own fp32 scores
    for src, ref_src in (("raw", logits_ref), ("group", group_ref)):
        dc.select(src=src)
        torch.cuda.synchronize()
        s_gpu = dc.host("scores")
        s_ref_src = oracle.aggregate(ref_src.astype(np.float32).astype(np.float64), c.prefix_len)
        _check(parity.score_gate(s_gpu, s_ref_src, mask=mask_s), f"select {src} scores")
        pr1, sr1, cr1 = oracle.topk(s_gpu.astype(np.float64), c.prefix_len, c.k, page_table=c.page_table,
                                    max_k=dc.max_k)
        cnt1 = dc.host("sel_count")
        _check(parity.exact_gate(cnt1, cr1), f"select {src} count")
        p1, q1 = dc.host("sel_pos"), dc.host("sel_slot")
        for b in range(c.batch):
            n = int(cr1[b])
            _check(parity.exact_gate(p1[b, :n], pr1[b, :n]), f"select {src} positions seq {b}")
            _check(parity.exact_gate(q1[b, :n], sr1[b, :n]), f"select {src} slots seq {b}")

    # top-k on the oracle's scores rounded to fp32: bit-exact against the oracle
    # taking the same decision in the same precision
    s_ref = oracle.aggregate(logits_ref, c.prefix_len)
    s32 = s_ref.astype(np.float32)
    dc.put("scores", s32)
    dc.topk()
    torch.cuda.synchronize()
    pos_ref, slot_ref, cnt_ref = oracle.topk(s32.astype(np.float64), c.prefix_len, c.k,
                                             page_table=c.page_table, max_k=dc.max_k)
    cnt = dc.host("sel_count")
    _check(parity.exact_gate(cnt, cnt_ref), "topk count")
    pos, slot = dc.host("sel_pos"), dc.host("sel_slot")
    for b in range(c.batch):
        n = int(cnt_ref[b])
        _check(parity.exact_gate(pos[b, :n], pos_ref[b, :n]), f"topk positions seq {b}")
        _check(parity.exact_gate(slot[b, :n], slot_ref[b, :n]), f"topk slots seq {b}")

    # sparse draft on the oracle's selection, every draft step's tail
    for s in range(c.gamma):
        dc.sel_slot.copy_(torch.from_numpy(slot_ref).cuda())
        dc.sel_count.copy_(torch.from_numpy(cnt_ref).cuda())
        dc.sparse(step=s)
        torch.cuda.synchronize()
        o_ref = oracle.sparse(np.ascontiguousarray(c.q_draft[s][:, None]), c.k_cache, c.v_cache,
                              c.page_table, pos_ref, cnt_ref, c.prefix_len,
                              np.full(c.batch, s + 1, np.int32), c.scale, nthreads=NTHREADS)
        _check(parity.output_gate(dc.host("draft_out"), o_ref), f"sparse draft step {s}")
    return dc, (out_ref, logits_ref, group_ref, s_ref)


def _run_chain(c, dc, refs, export):
    """End to end on the GPU's own intermediate results."""
    import torch
    out_ref, logits_ref, group_ref, s_ref = refs
    dc.iteration(export=export)
    torch.cuda.synchronize()
    _check(parity.output_gate(dc.host("out"), out_ref), f"chain[{export}] verify out")
    _check(parity.score_gate(dc.host("scores"), s_ref, mask=_rows_mask(c, ())), f"chain[{export}] scores")
    pos, cnt = dc.host("sel_pos"), dc.host("sel_count")
    _check(parity.topk_gate(pos, cnt, s_ref, c.prefix_len, c.k), f"chain[{export}] topk")
    slot = dc.host("sel_slot")
    for b in range(c.batch):
        n = int(cnt[b])
        p = pos[b, :n].astype(np.int64)
        expect = c.page_table[b, p // c.page_size].astype(np.int64) * c.page_size + p % c.page_size
        _check(parity.exact_gate(slot[b, :n], expect), f"chain[{export}] slot translation seq {b}")
    if c.gamma == 0:  # no draft steps
        return
    # last draft step, against the oracle over the GPU's own selection
    s = c.gamma - 1
    o_ref = oracle.sparse(np.ascontiguousarray(c.q_draft[s][:, None]), c.k_cache, c.v_cache,
                          c.page_table, pos, cnt, c.prefix_len, np.full(c.batch, s + 1, np.int32),
                          c.scale, nthreads=NTHREADS)
    _check(parity.output_gate(dc.host("draft_out"), o_ref), f"chain[{export}] sparse draft")


# ------------------------------------------------------------------ small cases

SMALL = {
    "c1_tiny": lambda: synth.CONFIGS["c1_tiny"],
    "c1_tiny_sharp": lambda: synth.sharp(synth.CONFIGS["c1_tiny"]),
    "c2_small": lambda: synth.small("c2_qwen3_32k", prefix=(3001,)),
    "c2_small_sharp": lambda: synth.sharp(synth.small("c2_qwen3_32k", prefix=(3001,))),
    "c3_small": lambda: synth.small("c3_qwen3_128k", prefix=(9000,), span_len=64),
    "c4_small": lambda: synth.small("c4_ragged_b8", prefix=(700, 1531, 4097)),
    "c5_small": lambda: synth.small("c5_gptoss_64k", prefix=(2000, 2077)),
    "c5_small_sharp": lambda: synth.sharp(synth.small("c5_gptoss_64k", prefix=(2000, 2077))),
    "short_prefixes": lambda: synth.small("c2_qwen3_32k", prefix=(1, 5, 17, 33), gamma=4, k_pct=50),
    "short_prefixes_g8": lambda: synth.small("c5_gptoss_64k", prefix=(3, 16, 31, 64), gamma=5, k_pct=50),
    # gamma = 0: the first draft row and the bonus row are the same row (counted twice)
    "gamma0": lambda: synth.small("c2_qwen3_32k", prefix=(1500, 1), gamma=0, k_pct=10),
    # one query head per KV head: plain decode attention
    "g1_decode": lambda: synth.small("c5_gptoss_64k", prefix=(3000, 700), num_q_heads=8, num_kv_heads=8,
                                     gamma=2),
    # the same at D = 128: two staged raw rows per KV head (8192-entry chunks)
    "g1_d128": lambda: synth.small("c2_qwen3_32k", prefix=(3000, 700), num_q_heads=8, num_kv_heads=8,
                                   gamma=2),
    # 64 ragged sequences under a permuted pool: many work-split segments
    "many_seqs": lambda: synth.small("c2_qwen3_32k", prefix=tuple(17 + (i * 613) % 1900 for i in range(64)),
                                     gamma=3, paging="permuted", ramp=0, spans=0),
    # 64 query rows per KV head at D = 128 (4 row tiles)
    "rows64_d128": lambda: synth.small("c2_qwen3_32k", prefix=(2100,), num_q_heads=64, num_kv_heads=8,
                                       gamma=7),
    # empty prefixes (P = 0): the new tokens only, nothing to export or select
    "empty_prefix": lambda: synth.small("c2_qwen3_32k", prefix=(0, 3000, 0, 40), gamma=4, k_pct=50),
    # every verify row-tile count at both head sizes: D = 128 with 3 row tiles
    # (36 rows), D = 64 with 2 and 4 row tiles (32 and 64 rows)
    "rows36_d128": lambda: synth.small("c2_qwen3_32k", prefix=(2500, 613), gamma=8),
    "rows32_d64": lambda: synth.small("c5_gptoss_64k", prefix=(2000, 1203), gamma=3),
    "rows64_d64": lambda: synth.small("c5_gptoss_64k", prefix=(2000, 2077, 45), gamma=7),
    # equal prefix lengths: with unpadded rows (max_prefix = P) the verify
    # combine keeps its speculative first loads
    "uniform_b3": lambda: synth.small("c5_gptoss_64k", prefix=(2077,) * 3),
    "uniform_b16": lambda: synth.small("c2_qwen3_32k", prefix=(700,) * 16, paging="permuted", ramp=0, spans=0),
    # keys rising along the sequence (a ramp over the whole prefix, no sink or
    # heavy hitters): the running maximum keeps growing from tile to tile, so
    # every rescale of the online softmax matters
    "rising": lambda: synth.small("c2_qwen3_32k", prefix=(3000, 1500), ramp=3000, sink=False, hh_pct=0,
                                  spans=0),
    # k = P: every prefix position selected
    "k_all": lambda: synth.small("c5_gptoss_64k", prefix=(300, 77), k_pct=100),
    # fp32 cache at D = 128 (the VALU kernel's other head size), ragged, permuted pool
    "f32_d128": lambda: synth.small("c4_ragged_b8", prefix=(1200, 333, 2049), dtype="f32"),
    # fp32 with G = 8 query heads per KV head at D = 64
    "f32_g8": lambda: synth.small("c5_gptoss_64k", prefix=(900, 1601), dtype="f32"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(torch_cuda, name):
    c = synth.make_case(SMALL[name]())
    dc, refs = _run_steps(c)
    _run_chain(c, dc, refs, "group")
    _run_chain(c, dc, refs, "raw")


@pytest.mark.parametrize("name", ["c4_small", "c5_small", "short_prefixes", "c2_small", "c3_small",
                                  "uniform_b3", "uniform_b16"])
def test_small_parity_unpadded_rows(torch_cuda, name):
    """Export / score rows exactly max_prefix floats long (unaligned strides).
    With equal prefix lengths this is also the verify combine's speculation on
    equal lengths taken (c2_small, c3_small, uniform_*) rather than dropped."""
    c = synth.make_case(SMALL[name]())
    dc, refs = _run_steps(c, pad=1)
    _run_chain(c, dc, refs, "group")
    _run_chain(c, dc, refs, "raw")


@pytest.mark.parametrize("name", ["c2_small", "c5_small", "short_prefixes", "rising"])
def test_small_parity_valu_bf16(torch_cuda, name):
    from verification_guided_sparse_amd import _binding as vg
    c = synth.make_case(SMALL[name]())
    _run_steps(c, kernel=vg.VG_KERNEL_VALU)


@pytest.mark.parametrize("base,kw,kernel", [
    ("c2_qwen3_32k", dict(prefix=(2500, 1200)), "auto"),           # MFMA, D = 128
    ("c5_gptoss_64k", dict(prefix=(2000, 3100)), "auto"),          # MFMA, D = 64, G = 8
    ("c4_ragged_b8", dict(prefix=(900, 2100), dtype="f32"), "auto"),  # VALU, fp32
    ("c2_qwen3_32k", dict(prefix=(2500, 1200)), "valu"),           # VALU, bf16
])
def test_page_permutation_bit_identical(torch_cuda, base, kw, kernel):
    """Same logical data under identity and permuted page tables: identical bits."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd.runner import DeviceCase
    cfg = synth.small(base, **kw)
    kern = {"auto": vg.VG_KERNEL_AUTO, "valu": vg.VG_KERNEL_VALU}[kernel]
    _say(f"[parity] page permutation {base} {kw} kernel={kernel}")
    res = []
    for paging in ("identity", "permuted"):
        c = synth.make_case(synth.dataclasses.replace(cfg, paging=paging))
        dc = DeviceCase(c, kernel=kern)
        dc.iteration(export="both")
        torch.cuda.synchronize()
        res.append((dc.host("out"), dc.host("logits"), dc.host("group"), dc.host("scores"),
                    dc.host("sel_pos"), dc.host("draft_out")))
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_bit_reproducible(torch_cuda):
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(synth.small("c5_gptoss_64k", prefix=(3000, 4100)))
    dc = DeviceCase(c)
    outs = []
    for _ in range(2):
        dc.iteration(export="raw")
        torch.cuda.synchronize()
        outs.append([dc.host(n).copy() for n in ("out", "logits", "scores", "sel_pos", "sel_slot", "draft_out")])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_topk_ties_and_edges(torch_cuda):
    """Integer-valued scores with many ties, k = 0, k > P, P = 0 and -0.0 vs +0.0."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    B, mp = 6, 5000
    rng = np.random.default_rng(11)
    s = rng.integers(-3, 4, size=(B, mp)).astype(np.float32)
    s[3, ::2] = -0.0
    s[3, 1::2] = 0.0
    P = np.array([5000, 4097, 0, 3000, 2048, 1], np.int32)
    k = np.array([2500, 0, 7, 1500, 2048, 5], np.int32)
    max_k = 2500
    pt = np.arange(B * 320, dtype=np.int32).reshape(B, 320)
    dev = dict(device="cuda")
    ts = torch.from_numpy(s).cuda()
    tP, tk, tpt = (torch.from_numpy(x).cuda() for x in (P, k, pt))
    pos = torch.full((B, max_k), -1, dtype=torch.int32, **dev)
    slot = torch.full((B, max_k), -1, dtype=torch.int32, **dev)
    cnt = torch.zeros(B, dtype=torch.int32, **dev)
    nbytes = vg.vg_topk_workspace_size(B, mp)
    ws = torch.empty(nbytes, dtype=torch.uint8, **dev)
    vg.vg_workspace_zero(ws, nbytes)
    for rep in range(2):  # the workspace must come back clean
        vg.vg_topk_select(B, ts, mp, tP, tk, max_k, tpt, 16, 320, pos, slot, cnt, 0, ws, nbytes)
        torch.cuda.synchronize()
        pr, sr, cr = oracle.topk(s.astype(np.float64), P, k, page_table=pt, max_k=max_k)
        assert np.array_equal(cnt.cpu().numpy(), cr)
        hp, hs = pos.cpu().numpy(), slot.cpu().numpy()
        for b in range(B):
            n = int(cr[b])
            assert np.array_equal(hp[b, :n], pr[b, :n]), (rep, b)
            assert np.array_equal(hs[b, :n], sr[b, :n]), (rep, b)


def test_out_of_range_counts_are_clamped(torch_cuda):
    """Device-side lengths the host cannot check are clamped to what the
    buffers were sized for, never turned into out-of-bounds accesses: top-k
    takes P_b in [0, max_prefix] and k_b in [0, min(P_b, max_k)]; the sparse
    draft takes sel_count in [0, max_k] and tail_len in [1, max_tail]."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd.runner import DeviceCase, _dev
    # top-k
    B, mp, max_k = 4, 3000, 400
    rng = np.random.default_rng(5)
    s = rng.standard_normal((B, mp)).astype(np.float32)
    P = np.array([3000, 5000, -5, 1000], np.int32)  # 5000 > max_prefix, -5 < 0
    k = np.array([900, 200, 5, -3], np.int32)         # 900 > max_k, -3 < 0
    pt = np.arange(B * 200, dtype=np.int32).reshape(B, 200)
    ts, tP, tk, tpt = (torch.from_numpy(x).cuda() for x in (s, P, k, pt))
    pos = torch.full((B, max_k), -1, dtype=torch.int32, device="cuda")
    slot = torch.full((B, max_k), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    nbytes = vg.vg_topk_workspace_size(B, mp)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    vg.vg_workspace_zero(ws, nbytes)
    vg.vg_topk_select(B, ts, mp, tP, tk, max_k, tpt, 16, 200, pos, slot, cnt, 0, ws, nbytes)
    torch.cuda.synchronize()
    Pc = np.clip(P, 0, mp)
    kc = np.minimum(np.clip(k, 0, None), np.minimum(Pc, max_k)).astype(np.int32)
    pr, sr, cr = oracle.topk(s.astype(np.float64), Pc, kc, page_table=pt, max_k=max_k)
    assert np.array_equal(cnt.cpu().numpy(), kc)
    assert np.array_equal(cr, kc)
    hp, hs = pos.cpu().numpy(), slot.cpu().numpy()
    for b in range(B):
        n = int(kc[b])
        assert np.array_equal(hp[b, :n], pr[b, :n]), b
        assert np.array_equal(hs[b, :n], sr[b, :n]), b
        assert np.all(hp[b, n:] == -1), b  # nothing written past the count

    # sparse draft: a full list of max_k valid slots, sel_count past max_k,
    # tail_len past max_tail
    c = synth.make_case(synth.small("c2_qwen3_32k", prefix=(3001, 1200)))
    dc = DeviceCase(c)
    mk = dc.max_k
    sel = np.stack([np.sort(rng.choice(int(c.prefix_len[b]), size=mk, replace=False))
                    for b in range(c.batch)]).astype(np.int32)
    slots = (c.page_table[np.arange(c.batch)[:, None], sel // 16] * 16 + sel % 16).astype(np.int32)
    over_cnt = np.full(c.batch, mk + 100, np.int32)
    over_tail = np.full(c.batch, dc.max_tail + 3, np.int32)
    dc.sparse(step=0, sel_slot=_dev(slots, dc.device), sel_count=_dev(over_cnt, dc.device),
              tail_len=_dev(over_tail, dc.device))
    torch.cuda.synchronize()
    want = oracle.sparse(np.ascontiguousarray(c.q_draft[0][:, None]), c.k_cache, c.v_cache, c.page_table,
                         sel, np.full(c.batch, mk, np.int32), c.prefix_len,
                         np.full(c.batch, dc.max_tail, np.int32), c.scale, nthreads=NTHREADS)
    _check(parity.output_gate(dc.host("draft_out"), want), "sparse draft with clamped counts")


@pytest.mark.parametrize("name,kernel", [("c2_qwen3_32k", "auto"), ("c5_gptoss_64k", "auto"),
                                         ("c2_qwen3_32k", "valu"), ("c1_tiny", "auto")])
def test_single_key_gather_is_exact(torch_cuda, name, kernel):
    """A row that sees exactly one key has softmax weight 1 on it, so its output
    is that key's value row converted to fp32, bit for bit: verify row 0 over
    an empty prefix, and a draft step over a one-entry tail with nothing
    selected.  This checks the gathers through the page table and the
    normalisation of both kernels exactly."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(synth.small(name, prefix=(0, 0, 0), gamma=3, paging="permuted"))
    kern = {"auto": vg.VG_KERNEL_AUTO, "valu": vg.VG_KERNEL_VALU}[kernel]
    _say(f"[parity] single-key gather {name} kernel={kernel}")
    dc = DeviceCase(c, kernel=kern)
    dc.verify(export="group")
    dc.window(n_sink=0)  # k = 0 for an empty prefix: nothing selected
    dc.sparse(step=0)    # tail_len 1: position 0 only
    torch.cuda.synchronize()
    G = c.num_q_heads // c.num_kv_heads
    v = c.v_cache if c.dtype == "f32" else synth.bf16_bits_to_f32(c.v_cache)
    slot0 = c.page_table[:, 0].astype(np.int64) * 16  # position 0 of each sequence
    want = np.stack([np.repeat(v[slot0[b]], G, axis=0) for b in range(c.batch)])  # [B][Hq][D]
    assert np.array_equal(dc.host("sel_count"), np.zeros(c.batch, np.int32))
    assert np.array_equal(dc.host("out")[:, 0], want)
    assert np.array_equal(dc.host("draft_out")[:, 0], want)


@pytest.mark.parametrize("name,n_q,kernel", [("c2_small", 2, "auto"), ("c2_small", 5, "auto"),
                                              ("c3_small", 7, "auto"), ("c5_small", 3, "auto"),
                                              ("c5_small", 6, "auto"), ("c4_small", 4, "auto"),
                                              ("short_prefixes", 3, "auto"), ("c2_small", 3, "valu"),
                                              ("c1_tiny", 5, "auto")])
def test_sparse_multi_row_draft(torch_cuda, name, n_q, kernel):
    """Sparse attention for n_q > 1 query rows in one call: row j attends the
    selected positions and the tail up to its own position (tail_len - n_q + j + 1
    of the new tokens), so the rows share the selection and differ only in the
    causal tail.  A seeded random selection of k_b positions per sequence stands
    in for the top-k (the kernel sees only slots)."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd.runner import DeviceCase, _dev
    c = synth.make_case(SMALL[name]())
    R = c.rows
    assert 1 <= n_q <= R
    _say(f"[parity] sparse multi-row {name} n_q={n_q} kernel={kernel}")
    kern = {"auto": vg.VG_KERNEL_AUTO, "valu": vg.VG_KERNEL_VALU}[kernel]
    dc = DeviceCase(c, kernel=kern, max_tail=R)
    rng = np.random.default_rng(4242 + n_q)
    pos = np.full((c.batch, dc.max_k), -1, np.int32)
    cnt = np.zeros(c.batch, np.int32)
    for b in range(c.batch):
        P = int(c.prefix_len[b])
        kb = min(int(c.k[b]), P)
        pos[b, :kb] = np.sort(rng.choice(P, size=kb, replace=False))
        cnt[b] = kb
    slot = np.full_like(pos, -1)
    for b in range(c.batch):
        p = pos[b, :cnt[b]].astype(np.int64)
        slot[b, :cnt[b]] = c.page_table[b, p // c.page_size] * c.page_size + p % c.page_size
    q = np.ascontiguousarray(c.q[:, R - n_q:])  # the last n_q verify rows as draft rows
    tail_len = np.full(c.batch, R, np.int32)
    dev = dc.device
    out = torch.zeros(c.batch, n_q, c.num_q_heads, c.head_dim, dtype=torch.float32, device=dev)
    ws_bytes = vg.vg_sparse_draft_workspace_size(dc.shape, n_q, dc.max_k, R)
    ws = dc._workspace(ws_bytes)
    vg.vg_sparse_draft_attention(dc.shape, _dev(q, dev), n_q, dc.k_cache, dc.v_cache,
                                 _dev(slot, dev), _dev(cnt, dev), dc.max_k,
                                 dc.page_table, dc.tail_start, _dev(tail_len, dev), R,
                                 out, ws, ws_bytes)
    torch.cuda.synchronize()
    o_ref = oracle.sparse(q, c.k_cache, c.v_cache, c.page_table, pos, cnt, c.prefix_len, tail_len,
                          c.scale, nthreads=NTHREADS)
    _check(parity.output_gate(out.cpu().numpy(), o_ref), f"sparse multi-row n_q={n_q}")
    # the last row sees every new token, as a one-row call over the whole tail does
    out1 = torch.zeros(c.batch, 1, c.num_q_heads, c.head_dim, dtype=torch.float32, device=dev)
    ws1_bytes = vg.vg_sparse_draft_workspace_size(dc.shape, 1, dc.max_k, R)
    ws1 = dc._workspace(ws1_bytes)
    vg.vg_sparse_draft_attention(dc.shape, _dev(q[:, -1:], dev), 1,
                                 dc.k_cache, dc.v_cache, _dev(slot, dev),
                                 _dev(cnt, dev), dc.max_k, dc.page_table, dc.tail_start,
                                 _dev(tail_len, dev), R, out1, ws1, ws1_bytes)
    torch.cuda.synchronize()
    _check(parity.output_gate(out1.cpu().numpy(), o_ref[:, -1:]), "sparse one-row call, whole tail")


def _topk_cases():
    """(name, scores [B][mp] f32, P, k, max_k): edge and tie cases inside the
    one-launch selection's range (max_prefix <= 2^17, even)."""
    rng = np.random.default_rng(2024)
    out = []
    mp = 131072
    # integer scores: tens of thousands of candidates share the threshold
    # bin (past the LDS candidate cache), heavy ties at K*
    s = rng.integers(0, 4, size=(2, mp)).astype(np.float32)
    out.append(("heavy_ties", s, np.array([mp, 99_999], np.int32), np.array([40_000, 7], np.int32), 40_000))
    # 1/64 grid: moderate ties
    s = (np.round(rng.standard_normal((3, mp)) * 64) / 64).astype(np.float32)
    out.append(("moderate_ties", s, np.array([mp, 70_001, 2049], np.int32),
                np.array([5243, 3500, 2049], np.int32), 5243))
    # continuous scores with a few exact copies of a value just above the k-th
    # largest, spread over several chunks: a small tie set at K* of which some
    # are taken (the resolve's ranked-list path)
    s = rng.standard_normal((2, mp)).astype(np.float32)
    P2, k2 = np.array([mp, 100_000], np.int32), np.array([5243, 777], np.int32)
    for b in range(2):
        t = np.sort(s[b, :P2[b]])[::-1][k2[b] - 5]
        s[b, rng.choice(P2[b], 7, replace=False)] = t
    out.append(("list_ties", s, P2, k2, 5243))
    # continuous scores, ragged lengths around chunk edges, k = 0, k > P, P = 0, P = 1
    s = rng.standard_normal((8, 8192)).astype(np.float32)
    s[6, ::2] = -0.0
    s[6, 1::2] = 0.0
    out.append(("ragged_edges", s, np.array([8192, 2048, 2049, 0, 1, 4097, 3000, 6000], np.int32),
                np.array([400, 0, 2049, 5, 1, 5000, 1500, 3], np.int32), 4097))
    return out


@pytest.mark.parametrize("case", [c[0] for c in _topk_cases()])
def test_topk_paths_agree(torch_cuda, case):
    """Every top-k path on the same fp32 scores, bit-exact against the oracle:
    vg_topk_select in one launch, the three-pass path (vg_aggregate_scores with
    the fused first pass, then VG_TOPK_PREPASS_DONE), and
    vg_aggregate_topk_select on a one-row export holding the scores; each run
    twice on one workspace (it must come back clean)."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    name, s, P, k, max_k = next(c for c in _topk_cases() if c[0] == case)
    B, mp = s.shape
    _say(f"[parity] top-k paths {name} B={B} mp={mp}")
    npg = -(-mp // 16)
    rng = np.random.default_rng(7)
    pt = np.stack([rng.permutation(npg) for _ in range(B)]).astype(np.int32)
    # (the GPU gets k as is and clamps it to max_k; the oracle takes k <= max_k)
    pr, sr, cr = oracle.topk(s.astype(np.float64), P, np.minimum(k, max_k), page_table=pt, max_k=max_k)
    dev = dict(device="cuda")
    ts = torch.from_numpy(s).cuda()
    tP, tk, tpt = (torch.from_numpy(x).cuda() for x in (P, k, pt))
    nbytes = vg.vg_topk_workspace_size(B, mp)
    ws = torch.empty(nbytes, dtype=torch.uint8, **dev)
    vg.vg_workspace_zero(ws, nbytes)
    scores = torch.zeros(B, mp, dtype=torch.float32, **dev)

    def run(path):
        pos = torch.full((B, max_k), -1, dtype=torch.int32, **dev)
        slot = torch.full((B, max_k), -1, dtype=torch.int32, **dev)
        cnt = torch.full((B,), -1, dtype=torch.int32, **dev)
        if path == "onepass":
            vg.vg_topk_select(B, ts, mp, tP, tk, max_k, tpt, 16, npg, pos, slot, cnt, 0, ws, nbytes)
        elif path == "threepass":
            vg.vg_aggregate_scores(B, ts, 1, 1, tP, mp, scores, ws, nbytes)
            vg.vg_topk_select(B, scores, mp, tP, tk, max_k, tpt, 16, npg, pos, slot, cnt,
                              vg.VG_TOPK_PREPASS_DONE, ws, nbytes)
        else:
            vg.vg_aggregate_topk_select(B, ts, 1, 1, tP, mp, scores, tk, max_k, tpt, 16, npg, pos, slot, cnt,
                                        ws, nbytes)
        torch.cuda.synchronize()
        return pos.cpu().numpy(), slot.cpu().numpy(), cnt.cpu().numpy()

    for path in ("onepass", "threepass", "fused", "onepass", "fused"):
        hp, hs, hc = run(path)
        assert np.array_equal(hc, cr), path
        for b in range(B):
            n = int(cr[b])
            assert np.array_equal(hp[b, :n], pr[b, :n]), (path, b)
            assert np.array_equal(hs[b, :n], sr[b, :n]), (path, b)
            assert np.all(hp[b, n:] == -1), (path, b)
        if path != "onepass":  # the scores written by the aggregation are the input, exactly
            sc = scores.cpu().numpy()
            for b in range(B):
                assert np.array_equal(sc[b, :P[b]], s[b, :P[b]]), (path, b)


def test_topk_moderate_ties(torch_cuda):
    """Scores on a 1/64 grid: tens to hundreds of positions share the k-th
    score (the last pass's short path through the threshold's tie group, as
    opposed to the long path the integer-score cases take); bit-exact."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    B, mp = 3, 300_000
    rng = np.random.default_rng(64)
    s = (np.round(rng.standard_normal((B, mp)) * 64) / 64).astype(np.float32)
    P = np.array([300_000, 123_457, 40_001], np.int32)
    k = np.array([15_000, 77_777, 2_001], np.int32)
    max_k = int(k.max())
    npg = -(-mp // 16)
    pt = np.stack([rng.permutation(npg) for _ in range(B)]).astype(np.int32)
    s64 = s.astype(np.float64)
    for b in range(B):  # the threshold value is shared by many positions
        kth = np.sort(s64[b, :P[b]])[::-1][k[b] - 1]
        assert 10 < int((s64[b, :P[b]] == kth).sum()) < 1024
    _say("[parity] top-k with moderate ties")
    dev = dict(device="cuda")
    ts = torch.from_numpy(s).cuda()
    tP, tk, tpt = (torch.from_numpy(x).cuda() for x in (P, k, pt))
    pos = torch.full((B, max_k), -1, dtype=torch.int32, **dev)
    slot = torch.full((B, max_k), -1, dtype=torch.int32, **dev)
    cnt = torch.zeros(B, dtype=torch.int32, **dev)
    nbytes = vg.vg_topk_workspace_size(B, mp)
    ws = torch.empty(nbytes, dtype=torch.uint8, **dev)
    vg.vg_workspace_zero(ws, nbytes)
    pr, sr, cr = oracle.topk(s64, P, k, page_table=pt, max_k=max_k)
    for rep in range(2):
        vg.vg_topk_select(B, ts, mp, tP, tk, max_k, tpt, 16, npg, pos, slot, cnt, 0, ws, nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(cnt.cpu().numpy(), cr)
        hp, hs = pos.cpu().numpy(), slot.cpu().numpy()
        for b in range(B):
            n = int(cr[b])
            assert np.array_equal(hp[b, :n], pr[b, :n]), (rep, b)
            assert np.array_equal(hs[b, :n], sr[b, :n]), (rep, b)


def test_topk_max_prefix(torch_cuda):
    """The longest score row the select kernels take (2^21 positions, 1024
    chunks), with so many ties at the threshold that the candidates overflow
    the LDS cache of the last pass; bit-exact, twice (the workspace comes back
    clean)."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    mp = 1 << 21
    _say(f"[parity] top-k at max_prefix={mp}")
    rng = np.random.default_rng(21)
    s = rng.integers(-3, 4, size=(1, mp)).astype(np.float32)
    P = np.array([mp], np.int32)
    k = np.array([mp // 2 + 12345], np.int32)
    max_k = int(k[0])
    npg = mp // 16
    pt = rng.permutation(npg).astype(np.int32)[None]
    dev = dict(device="cuda")
    ts = torch.from_numpy(s).cuda()
    tP, tk, tpt = (torch.from_numpy(x).cuda() for x in (P, k, pt))
    pos = torch.full((1, max_k), -1, dtype=torch.int32, **dev)
    slot = torch.full((1, max_k), -1, dtype=torch.int32, **dev)
    cnt = torch.zeros(1, dtype=torch.int32, **dev)
    nbytes = vg.vg_topk_workspace_size(1, mp)
    ws = torch.empty(nbytes, dtype=torch.uint8, **dev)
    vg.vg_workspace_zero(ws, nbytes)
    pr, sr, cr = oracle.topk(s.astype(np.float64), P, k, page_table=pt, max_k=max_k)
    for rep in range(2):
        vg.vg_topk_select(1, ts, mp, tP, tk, max_k, tpt, 16, npg, pos, slot, cnt, 0, ws, nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(cnt.cpu().numpy(), cr)
        assert np.array_equal(pos.cpu().numpy()[0], pr[0]), rep
        assert np.array_equal(slot.cpu().numpy()[0], sr[0]), rep


def test_max_batch_parity(torch_cuda):
    """The largest batch the attention calls take (1024 sequences: four rounds
    of the length scan, 2048 (sequence, KV head) lists), ragged short prefixes
    including empty ones; every step against the oracle."""
    pre = tuple(int(x) for x in np.random.default_rng(5).integers(0, 300, 1024))
    c = synth.make_case(synth.small("c2_qwen3_32k", prefix=pre, num_q_heads=8, num_kv_heads=2, gamma=3,
                                    ramp=0, spans=0, k_pct=20, paging="permuted"))
    dc, refs = _run_steps(c)
    _run_chain(c, dc, refs, "group")


@pytest.mark.parametrize("pad", [1, 64])
@pytest.mark.parametrize("wl,export,prefix", [
    ("c3_qwen3_128k", "both", (100003, 0, 61441)),
    ("c3_qwen3_128k", "group", (131071, 130001, 129007, 131000, 120007)),
    ("c5_gptoss_64k", "both", (131071, 130001, 129007, 120007, 131000)),
])
def test_staged_exports_multichunk(torch_cuda, pad, wl, export, prefix):
    """Exports staged in LDS over several chunks of one workgroup's piece,
    ragged lists whose pieces straddle (sequence, KV head) lists, and export
    rows whose stride is not a multiple of 4 floats (pad=1: the runs' scalar
    tails).  D = 128, raw and group export: 2048-entry chunks for the raw rows,
    and an empty sequence between two long ones.  D = 128, group export alone
    over five long sequences: about 20K entries per workgroup, so the
    long-chunk kernel runs over two 16384-entry chunks.  D = 64 (two
    workgroups per CU, raw rows stored per tile): about 10K entries per
    workgroup, two 8192-entry chunks of staged group sums.  Entries past each
    sequence's prefix length stay as they were (zero)."""
    from verification_guided_sparse_amd.runner import DeviceCase
    torch = torch_cuda
    c = synth.make_case(synth.small(wl, prefix=prefix, k_pct=2))
    _say(f"[parity] staged exports {wl} {export} P={list(c.prefix_len)} pad={pad}")
    dc = DeviceCase(c, pad=pad)
    out_ref, logits_ref, group_ref = _oracle_all(c)
    dc.verify(export=export)
    torch.cuda.synchronize()
    _check(parity.output_gate(dc.host("out"), out_ref), "verify out")
    logits, group = dc.host("logits"), dc.host("group")
    if export == "both":
        _check(parity.score_gate(logits, logits_ref, mask=_rows_mask(c, (2, c.num_q_heads))), "verify logits")
    else:
        assert not logits.any(), "raw export written without a raw-export call"
    _check(parity.score_gate(group, group_ref, mask=_rows_mask(c, (c.num_kv_heads,))), "verify group scores")
    for b, P in enumerate(c.prefix_len):
        assert not logits[b, :, :, P:].any(), f"raw export written past the prefix of sequence {b}"
        assert not group[b, :, P:].any(), f"group export written past the prefix of sequence {b}"


@pytest.mark.parametrize("name,export", [("c2_small", "both"), ("c5_small", "group"), ("c4_small", "raw")])
def test_cache_bases_at_any_16_byte_offset(torch_cuda, name, export):
    """The kernels take any 16-byte-aligned K and V cache bases (the placement
    the runner uses only speeds them up): with the caches moved to other
    offsets into their allocations, a whole iteration (verify with its
    exports, aggregation, top-k, every draft step) gives bit-identical
    results."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(SMALL[name]())
    _say(f"[parity] cache base offsets {name} export={export}")
    dc = DeviceCase(c)
    names = ["out", "scores", "sel_pos", "sel_slot", "sel_count", "draft_out"]
    names += {"both": ["logits", "group"], "group": ["group"], "raw": ["logits"]}[export]

    def run():
        if export == "both":
            dc.verify(export="both")
            dc.select(src="group")
            for s in range(c.gamma):
                dc.sparse(step=s)
        else:
            dc.iteration(export=export)
        torch.cuda.synchronize()
        return {n: dc.host(n).copy() for n in names}

    def rebase(t, off):  # a copy of t starting `off` bytes into a fresh allocation
        buf = torch.empty(t.numel() * t.element_size() + off, dtype=torch.uint8, device=t.device)
        v = buf[off:].view(t.dtype).view(t.shape)
        v.copy_(t)
        return v

    ref = run()
    for k_off, v_off in ((16, 48), (4112, 0), (0, 0)):
        dc.k_cache, dc.v_cache = rebase(dc.k_cache, k_off), rebase(dc.v_cache, v_off)
        got = run()
        for n in names:
            assert np.array_equal(got[n], ref[n]), f"{n} differs with K at +{k_off}, V at +{v_off}"


# ------------------------------------------------------------------ full sizes

@pytest.mark.parametrize("name", ["c1_tiny", "c2_qwen3_32k", "c3_qwen3_128k", "c5_gptoss_64k", "c4_ragged_b8"])
def test_full_size_parity(torch_cuda, name):
    """Every workload at its full size, in the launch configuration the benchmark times."""
    c = synth.make_case(name)
    dc, refs = _run_steps(c)
    _run_chain(c, dc, refs, "group")


def test_graph_replay_matches_eager(torch_cuda):
    """One iteration captured in a HIP graph and replayed several times, with eager
    work and synchronisations between replays: every replay equals the eager run."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(synth.small("c5_gptoss_64k", prefix=(2500, 1200)))
    dc = DeviceCase(c)
    names = ("out", "group", "scores", "sel_pos", "sel_slot", "sel_count", "draft_out")
    dc.iteration(export="group")
    torch.cuda.synchronize()
    eager = [dc.host(n).copy() for n in names]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dc.iteration(export="group")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dc.iteration(export="group")
    torch.cuda.synchronize()
    for rep in range(3):
        for n in names:
            getattr(dc, n).fill_(-7)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {n: dc.host(n) for n in names}
        ref = dict(zip(names, eager))
        for n in ("out", "sel_count", "draft_out"):
            assert np.array_equal(got[n], ref[n]), (rep, n)
        for b in range(c.batch):  # entries the contract writes
            P, k = int(c.prefix_len[b]), int(ref["sel_count"][b])
            assert np.array_equal(got["group"][b, :, :P], ref["group"][b, :, :P]), (rep, b)
            assert np.array_equal(got["scores"][b, :P], ref["scores"][b, :P]), (rep, b)
            assert np.array_equal(got["sel_pos"][b, :k], ref["sel_pos"][b, :k]), (rep, b)
            assert np.array_equal(got["sel_slot"][b, :k], ref["sel_slot"][b, :k]), (rep, b)


@pytest.mark.parametrize("name,pad", [("c2_small", 64), ("c4_small", 64), ("c5_small", 64), ("short_prefixes", 64),
                                      ("c1_tiny", 64), ("c3_small", 64), ("c4_small", 1), ("c5_small", 1)])
def test_verify_select_matches_separate_calls(torch_cuda, name, pad):
    """vg_verify_select (verify with the group export, aggregation and top-k,
    the selection's staging in the combine's launch) gives bit for bit what
    vg_verify_attention followed by vg_aggregate_topk_select gives -- also on
    unpadded rows, where it runs the separate calls' kernels -- and the chain
    passes the oracle's gates."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(SMALL[name]())
    _say(f"[parity] verify_select {name} pad={pad}")
    dc = DeviceCase(c, pad=pad)
    dc.verify(export="group")
    dc.select(src="group")
    torch.cuda.synchronize()
    names = ("out", "group", "scores", "sel_pos", "sel_slot", "sel_count")
    ref = {n: dc.host(n).copy() for n in names}
    for n in ("out", "group", "scores"):
        getattr(dc, n).fill_(float("nan"))
    for n in ("sel_pos", "sel_slot", "sel_count"):
        getattr(dc, n).fill_(-7)
    for rep in range(2):
        dc.verify_select()
        torch.cuda.synchronize()
        for n in names:
            got = dc.host(n)
            if n in ("sel_pos", "sel_slot"):
                for b in range(c.batch):
                    m = int(ref["sel_count"][b])
                    assert np.array_equal(got[b, :m], ref[n][b, :m]), (n, b, rep)
            elif n in ("group", "scores"):
                mask = _rows_mask(c, (c.num_kv_heads,) if n == "group" else ())
                assert np.array_equal(np.where(mask, got, 0), np.where(mask, ref[n], 0)), (n, rep)
            else:
                assert np.array_equal(got, ref[n]), (n, rep)
    out_ref, logits_ref, group_ref = _oracle_all(c)
    s_ref = oracle.aggregate(logits_ref, c.prefix_len)
    _check(parity.output_gate(dc.host("out"), out_ref), "verify_select out")
    _check(parity.score_gate(dc.host("scores"), s_ref, mask=_rows_mask(c, ())), "verify_select scores")
    _check(parity.topk_gate(dc.host("sel_pos"), dc.host("sel_count"), s_ref, c.prefix_len, c.k),
           "verify_select topk")


@pytest.mark.parametrize("name", ["c2_small", "c5_small", "short_prefixes", "gamma0", "c1_tiny"])
def test_full_collection_parity(torch_cuda, name):
    """All-rows export (the objective over every verify row): logits of every row,
    group sums over every row, aggregation over gamma+1 rows, and the chain."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(SMALL[name]())
    _say(f"[parity] full collection {c.cfg.name}")
    out_ref, _, _, lall = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len, c.gamma,
                                        c.scale, export="all", nthreads=NTHREADS)
    grp_ref = oracle.group_sums(lall, c.num_kv_heads)
    dc = DeviceCase(c)
    dc.verify(export="both", rows="all")
    torch.cuda.synchronize()
    _check(parity.output_gate(dc.host("out"), out_ref), "verify out")
    _check(parity.score_gate(dc.host("logits_all"), lall, mask=_rows_mask(c, (c.rows, c.num_q_heads))),
           "all-rows logits")
    _check(parity.score_gate(dc.host("group"), grp_ref, mask=_rows_mask(c, (c.num_kv_heads,))),
           "all-rows group sums")
    # aggregation over gamma+1 rows, on the oracle's logits rounded to fp32
    l32 = lall.astype(np.float32)
    dc.put("logits_all", l32)
    dc.aggregate(src="raw_all")
    torch.cuda.synchronize()
    s_ref = oracle.aggregate(l32.astype(np.float64), c.prefix_len)
    _check(parity.score_gate(dc.host("scores"), s_ref, mask=_rows_mask(c, ())), "aggregate all rows")
    # chain, both export forms
    s_all = oracle.aggregate(lall, c.prefix_len)
    for export in ("raw", "group"):
        dc.iteration(export=export, rows="all")
        torch.cuda.synchronize()
        _check(parity.score_gate(dc.host("scores"), s_all, mask=_rows_mask(c, ())), f"chain[{export}] scores")
        _check(parity.topk_gate(dc.host("sel_pos"), dc.host("sel_count"), s_all, c.prefix_len, c.k),
               f"chain[{export}] topk")


@pytest.mark.parametrize("name", ["c4_small", "c1_tiny", "c5_small"])
def test_kv_append_bit_exact(torch_cuda, name):
    """The new tokens' rows written into a cache whose new-token slots were cleared:
    bit-identical to the oracle's append (and to the generated cache); positions
    outside the page-table row are skipped; the chain then verifies as usual."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd.runner import DeviceCase, _dev
    c = synth.make_case(SMALL[name]())
    R = c.rows
    pos = [np.arange(int(c.prefix_len[b]), int(c.prefix_len[b]) + R) for b in range(c.batch)]
    slots = [c.page_table[b, p // 16].astype(np.int64) * 16 + p % 16 for b, p in enumerate(pos)]
    k_new = np.stack([c.k_cache[s] for s in slots])  # [B][R][Hkv][D] raw
    v_new = np.stack([c.v_cache[s] for s in slots])
    k0, v0 = c.k_cache.copy(), c.v_cache.copy()
    for s in slots:
        k0[s] = 0
        v0[s] = 0
    k_ref, v_ref = oracle.kv_append(k0, v0, k_new, v_new, c.page_table, c.prefix_len)
    assert np.array_equal(k_ref, c.k_cache) and np.array_equal(v_ref, c.v_cache)
    _say(f"[parity] kv append {c.cfg.name}")
    dc = DeviceCase(c)
    # raw element bits both ways (bf16 travels as int16; the host side is uint16)
    up = lambda a: _dev(a, "cuda")
    down = lambda t, like: t.cpu().numpy().view(like.dtype)
    dc.k_cache.copy_(up(k0))
    dc.v_cache.copy_(up(v0))
    tk, tv = up(k_new), up(v_new)
    vg.vg_kv_append(dc.shape, tk, tv, R, dc.page_table, dc.prefix_len, dc.k_cache, dc.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(down(dc.k_cache, k_ref), k_ref)
    assert np.array_equal(down(dc.v_cache, v_ref), v_ref)
    # start positions past every page-table row: nothing is written
    far = torch.full_like(dc.prefix_len, dc.max_pages * 16)
    vg.vg_kv_append(dc.shape, tk, tv, R, dc.page_table, far, dc.k_cache, dc.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(down(dc.k_cache, k_ref), k_ref)
    # the appended cache verifies like the generated one
    out_ref, _, group_ref = _oracle_all(c)
    dc.verify(export="group")
    torch.cuda.synchronize()
    _check(parity.output_gate(dc.host("out"), out_ref), "verify after append")
    _check(parity.score_gate(dc.host("group"), group_ref, mask=_rows_mask(c, (c.num_kv_heads,))),
           "group after append")


@pytest.mark.parametrize("name", ["c4_small", "c5_small", "short_prefixes", "c1_tiny"])
def test_iterations_on_device(torch_cuda, name):
    """Several iterations with the cache, the prefix lengths and the selection kept on
    the device: append the new tokens, verify (group export), aggregate, top-k, the
    draft steps, then keep the accepted tokens.  Each iteration against the oracle run
    on a host copy of the same state; the cache and the lengths bit-exact."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase, _dev
    c = synth.make_case(SMALL[name]())
    R, n_iter = c.rows, 3
    p = (c.prefix_len - n_iter * R).astype(np.int32)  # the pages cover prefix_len + R
    p = np.maximum(p, 0)
    _say(f"[parity] iterations {c.cfg.name} start P={list(p)} gamma={c.gamma}")
    dc = DeviceCase(c)
    dc.prefix_len.copy_(torch.from_numpy(p))
    k_host, v_host = c.k_cache.copy(), c.v_cache.copy()
    down = lambda t, like: t.cpu().numpy().view(like.dtype)
    for it in range(n_iter):
        k_new, v_new = synth.new_token_rows(c, it)
        dc.append(_dev(k_new, "cuda"), _dev(v_new, "cuda"))
        k_host, v_host = oracle.kv_append(k_host, v_host, k_new, v_new, c.page_table, p)
        dc.verify(export="group")
        dc.aggregate(src="group", fuse_prepass=True)
        dc.topk(prepass_done=True)
        dc.sparse(step=c.gamma - 1, tail_start=dc.prefix_len) if c.gamma else None
        torch.cuda.synchronize()
        out_ref, _, group_ref, _ = oracle.verify(c.q, k_host, v_host, c.page_table, p, c.gamma, c.scale,
                                                 max_prefix=c.max_prefix, nthreads=NTHREADS)
        what = f"iteration {it}"
        _check(parity.output_gate(dc.host("out"), out_ref), f"{what} verify out")
        _check(parity.score_gate(dc.host("group"), group_ref,
                                 mask=parity.prefix_mask(p, c.max_prefix, (c.num_kv_heads,))), f"{what} group")
        s_ref = oracle.aggregate(group_ref, p)
        pos, cnt = dc.host("sel_pos"), dc.host("sel_count")
        _check(parity.topk_gate(pos, cnt, s_ref, p, c.k), f"{what} topk")
        if c.gamma:
            s = c.gamma - 1
            o_ref = oracle.sparse(np.ascontiguousarray(c.q_draft[s][:, None]), k_host, v_host, c.page_table,
                                  pos, cnt, p, np.full(c.batch, s + 1, np.int32), c.scale, nthreads=NTHREADS)
            _check(parity.output_gate(dc.host("draft_out"), o_ref), f"{what} sparse draft")
        n = synth.accepted_counts(c, it)
        dc.advance(_dev(n, "cuda"))
        p = oracle.advance_prefix(p, n, c.gamma)
        torch.cuda.synchronize()
        _check(parity.exact_gate(dc.host("prefix_len"), p), f"{what} prefix lengths")
    assert np.array_equal(down(dc.k_cache, k_host), k_host)
    assert np.array_equal(down(dc.v_cache, v_host), v_host)


@pytest.mark.parametrize("name", ["c4_small", "c5_small", "short_prefixes", "empty_prefix"])
@pytest.mark.parametrize("n_sink", [0, 4])
def test_window_select_and_draft(torch_cuda, name, n_sink):
    """The query-agnostic selection, bit-exact against the oracle, then every draft
    step through the same sparse kernel over it."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    c = synth.make_case(SMALL[name]())
    _say(f"[parity] window select {c.cfg.name} n_sink={n_sink} k={list(c.k)}")
    dc = DeviceCase(c)
    dc.window(n_sink=n_sink)
    torch.cuda.synchronize()
    pos_ref, slot_ref, cnt_ref = oracle.window_select(c.prefix_len, c.k, n_sink, c.page_table, max_k=dc.max_k)
    cnt = dc.host("sel_count")
    _check(parity.exact_gate(cnt, cnt_ref), "window count")
    pos, slot = dc.host("sel_pos"), dc.host("sel_slot")
    for b in range(c.batch):
        n = int(cnt_ref[b])
        _check(parity.exact_gate(pos[b, :n], pos_ref[b, :n]), f"window positions seq {b}")
        _check(parity.exact_gate(slot[b, :n], slot_ref[b, :n]), f"window slots seq {b}")
    for s in range(c.gamma):
        dc.sparse(step=s)
        torch.cuda.synchronize()
        o_ref = oracle.sparse(np.ascontiguousarray(c.q_draft[s][:, None]), c.k_cache, c.v_cache,
                              c.page_table, pos_ref, cnt_ref, c.prefix_len,
                              np.full(c.batch, s + 1, np.int32), c.scale, nthreads=NTHREADS)
        _check(parity.output_gate(dc.host("draft_out"), o_ref), f"draft over the window, step {s}")
