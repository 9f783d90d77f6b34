"""The C-ABI library on the CPU: it loads, exports every declared symbol, sizes
workspaces and rejects invalid arguments before touching the GPU."""
from __future__ import annotations

import ctypes as C
import os
import re

import pytest

from verification_guided_sparse_amd import _binding as vg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vegas_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vg_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = vg.lib()
    names = _declared()
    assert set(names) == set(vg.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert vg.status_string(vg.VG_OK) == "VG_OK"
    assert vg.status_string(vg.VG_ERR_WORKSPACE) == "VG_ERR_WORKSPACE"
    assert vg.status_string(99) == "VG_ERR_UNKNOWN"
    assert "gfx950" in vg.version()


def _shape(**kw):
    d = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_pages_per_seq=8200,
             dtype=vg.VG_DTYPE_BF16)
    d.update(kw)
    return vg.make_shape(**d)


def test_workspace_sizes():
    a = vg.vg_verify_workspace_size(_shape(), 131072, 6)
    b = vg.vg_verify_workspace_size(_shape(), 32768, 6)
    assert a > 0 and b > 0
    assert vg.vg_topk_workspace_size(8, 131072) > vg.vg_topk_workspace_size(1, 131072)
    assert vg.vg_sparse_draft_workspace_size(_shape(), 1, 5243, 7) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), vg.VG_ERR_UNSUPPORTED),
    (dict(num_q_heads=30), vg.VG_ERR_INVALID_ARG),
    (dict(dtype=7), vg.VG_ERR_INVALID_ARG),
    (dict(dtype=vg.VG_DTYPE_F32, kernel=vg.VG_KERNEL_MFMA), vg.VG_ERR_UNSUPPORTED),
    (dict(page_size=8), vg.VG_ERR_UNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=8), vg.VG_ERR_UNSUPPORTED),  # (gamma+1)*G > 64
])
def test_verify_size_rejects(kw, status):
    with pytest.raises(vg.VgError) as e:
        vg.vg_verify_workspace_size(_shape(**kw), 1024, 6)
    assert e.value.status == status


def test_verify_rejects_before_launch():
    """Invalid arguments return an error without any device work (runs on a CPU-only host)."""
    sh = _shape(max_pages_per_seq=100)
    fake = 0x10000  # 16-byte aligned, never dereferenced on these paths
    args = [fake] * 5
    # null output
    with pytest.raises(vg.VgError) as e:
        vg.vg_verify_attention(sh, *args, 1000, 4, None, None, None, fake, 1 << 30, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    # misaligned q
    with pytest.raises(vg.VgError) as e:
        vg.vg_verify_attention(sh, fake + 4, *args[1:], 1000, 4, fake, fake, None, fake, 1 << 30, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    # page table too short for max_prefix + gamma + 1
    with pytest.raises(vg.VgError) as e:
        vg.vg_verify_attention(sh, *args, 1600, 4, fake, fake, None, fake, 1 << 30, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    # gamma out of range
    with pytest.raises(vg.VgError) as e:
        vg.vg_verify_attention(sh, *args, 100, 16, fake, fake, None, fake, 1 << 30, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    # workspace too small
    need = vg.vg_verify_workspace_size(sh, 1000, 4)
    with pytest.raises(vg.VgError) as e:
        vg.vg_verify_attention(sh, *args, 1000, 4, fake, fake, None, fake, need - 1, 0)
    assert e.value.status == vg.VG_ERR_WORKSPACE


def test_topk_and_sparse_reject_before_launch():
    fake = 0x10000
    need = vg.vg_topk_workspace_size(2, 5000)
    with pytest.raises(vg.VgError) as e:  # bad flags
        vg.vg_topk_select(2, fake, 5000, fake, fake, 100, fake, 16, 400, fake, fake, fake, 5, fake, need, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    with pytest.raises(vg.VgError) as e:  # workspace too small
        vg.vg_topk_select(2, fake, 5000, fake, fake, 100, fake, 16, 400, fake, fake, fake, 0, fake, need - 16, 0)
    assert e.value.status == vg.VG_ERR_WORKSPACE
    with pytest.raises(vg.VgError) as e:  # page table too short for the slots
        vg.vg_topk_select(2, fake, 5000, fake, fake, 100, fake, 16, 300, fake, fake, fake, 0, fake, need, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    with pytest.raises(vg.VgError) as e:  # max_prefix above 2^21
        vg.vg_topk_workspace_size(1, (1 << 21) + 1)
    assert e.value.status == vg.VG_ERR_UNSUPPORTED
    sh = _shape()
    with pytest.raises(vg.VgError) as e:  # tail bound below n_q
        vg.vg_sparse_draft_attention(sh, fake, 2, fake, fake, fake, fake, 10, fake, fake, fake, 1, fake, fake, 1 << 30, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG
    with pytest.raises(vg.VgError) as e:  # null sel_slot with max_k > 0
        vg.vg_sparse_draft_attention(sh, fake, 1, fake, fake, None, fake, 10, fake, fake, fake, 2, fake, fake, 1 << 30, 0)
    assert e.value.status == vg.VG_ERR_INVALID_ARG


def test_batch_limit_and_long_lists():
    """Batches above the work-sharing table's capacity (1024 sequences) are
    reported before any launch; long key lists are accepted (the workgroups
    share tiles, so list length sets no limit)."""
    sh = _shape(batch=1025, max_pages_per_seq=1 << 20)
    for call in (lambda: vg.vg_sparse_draft_workspace_size(sh, 1, 100, 8),
                 lambda: vg.vg_verify_workspace_size(sh, 4096, 3)):
        with pytest.raises(vg.VgError) as e:
            call()
        assert e.value.status == vg.VG_ERR_UNSUPPORTED
    sh = _shape(max_pages_per_seq=1 << 20)
    assert vg.vg_sparse_draft_workspace_size(sh, 1, 600_000, 8) > 0
    assert vg.vg_verify_workspace_size(sh, 1 << 21, 7) > 0
