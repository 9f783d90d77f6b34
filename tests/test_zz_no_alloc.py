"""The sparse draft entry point that allocates nothing, against the one that
takes a caller workspace: bit-identical outputs on two calls in a row, the
second with a smaller input, and a clean refusal past the built-in array's size.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from tests import parity
from verification_guided_sparse_amd import synth

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    from verification_guided_sparse_amd import _binding
    _binding.lib()
    return torch


def _draft_both(dc, step):
    """Draft step `step` through both entry points; returns (with workspace, without)."""
    import torch
    from verification_guided_sparse_amd import _binding as vg
    dc.sparse(step=step)
    ref = dc.draft_out.clone()
    out = torch.full_like(ref, float("nan"))
    vg.vg_sparse_draft_attention_noalloc(
        dc.shape, dc.q_draft[step], 1, dc.k_cache, dc.v_cache, dc.sel_slot, dc.sel_count, dc.max_k,
        dc.page_table, dc.tail_start, dc.tail_len[step], dc.max_tail, out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_draft_matches_workspace_entry(torch_cuda):
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    # a larger call, then a smaller one: the second must not see the first's partials
    cases = [synth.small("c5_gptoss_64k", prefix=(20000, 15000)),
             synth.small("c2_qwen3_32k", prefix=(3001,))]
    for cfg in cases:
        c = synth.make_case(cfg)
        print(f"[no-alloc] {c.cfg.name} B={c.batch} P={list(c.prefix_len)} G={c.num_q_heads // c.num_kv_heads} "
              f"D={c.head_dim}", flush=True)
        dc = DeviceCase(c)
        dc.iteration(export="group")  # a selection for the draft steps
        torch.cuda.synchronize()
        for step in (c.gamma - 1, 0):
            ref, out = _draft_both(dc, step)
            assert torch.equal(ref, out), f"{c.cfg.name} step {step}: outputs differ"
        # and the parity bar against the oracle, on the GPU's own selection
        pos, cnt = dc.host("sel_pos"), dc.host("sel_count")
        want = oracle.sparse(np.ascontiguousarray(c.q_draft[0][:, None]), c.k_cache, c.v_cache, c.page_table,
                             pos, cnt, c.prefix_len, np.full(c.batch, 1, np.int32), c.scale,
                             nthreads=NTHREADS)
        ok, msg = parity.output_gate(out.cpu().numpy(), want)
        assert ok, msg


def test_noalloc_refuses_oversize(torch_cuda):
    import torch
    from verification_guided_sparse_amd import _binding as vg
    shape = vg.make_shape(8, 32, 8, 128, 1 << 16, vg.VG_DTYPE_BF16, 0.0, vg.VG_KERNEL_AUTO, 16)
    need = vg.vg_sparse_draft_workspace_size(shape, 1, 1 << 20, 8)
    assert need > vg.VG_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(vg.VgError) as e:
        vg.vg_sparse_draft_attention_noalloc(shape, dummy, 1, dummy, dummy, dummy, dummy, 1 << 20, dummy,
                                             dummy, dummy, 8, dummy)
    assert e.value.status == vg.VG_ERR_WORKSPACE
    assert torch.count_nonzero(dummy).item() == 0  # nothing launched
