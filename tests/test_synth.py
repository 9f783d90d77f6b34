"""The seeded generator: deterministic, shaped and structured as configured."""
from __future__ import annotations

import hashlib

import numpy as np

from verification_guided_sparse_amd import synth


def _digest(case):
    h = hashlib.sha256()
    for a in (case.q, case.q_draft, case.k_cache, case.v_cache, case.page_table, case.prefix_len, case.k):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic():
    cfg = synth.small("c4_ragged_b8", prefix=(300, 1000, 17))
    assert _digest(synth.make_case(cfg)) == _digest(synth.make_case(cfg))
    assert _digest(synth.make_case(cfg)) != _digest(synth.make_case(cfg, seed=cfg.seed + 1))


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even (down)
    assert back[2] == 1.0 + 4 * 2**-8          # tie -> even (up)
    assert back[3] == -2.5
    assert np.all(np.abs(back[:5] - x[:5]) <= np.abs(x[:5]) * 2**-8)
    assert abs(float(back[5]) - 1e-40) <= 2.0**-133  # subnormal: absolute half-ulp


def test_c1_shapes_and_structure():
    c = synth.make_case("c1_tiny")
    assert c.q.shape == (1, 5, 8, 64) and c.q.dtype == np.float32
    assert c.k_cache.shape[1:] == (2, 64)
    assert int(c.k[0]) == 205 and int(c.prefix_len[0]) == 2048
    assert len(c.heavy[0]) == 41 and 0 not in c.heavy[0]
    # identity paging, -1 past the last page
    n_pages = -(-(2048 + 5) // 16)
    assert np.array_equal(c.page_table[0, :n_pages], np.arange(n_pages))
    # heavy hitters stand out along the seeded direction: K . u is ~3 there and ~0 elsewhere
    u = synth._unit_vectors(c.cfg.seed, 0, 2, 64)
    proj = np.einsum("jgd,gd->jg", c.k_cache[:2048].astype(np.float64), u)
    hh = np.zeros(2048, bool)
    hh[c.heavy[0]] = True
    hh[0] = True
    assert np.all(proj[hh] > 2.0) and np.all(np.abs(proj[~hh]) < 1.5)


def test_c3_spans_and_ramp_small():
    cfg = synth.small("c3_qwen3_128k", prefix=(8192,), span_len=16)
    c = synth.make_case(cfg)
    h = c.heavy[0]
    assert len(h) == synth.pct_round_half_up(8192, 1)
    runs = np.split(h, np.flatnonzero(np.diff(h) != 1) + 1)
    assert sum(1 for r in runs if len(r) >= 16) == 3
    u = synth._unit_vectors(cfg.seed, 0, 8, 128)
    K = synth.bf16_bits_to_f32(c.k_cache[:8192]).astype(np.float64)
    proj = np.einsum("jgd,gd->jg", K, u).mean(axis=1)
    # recency ramp: projection rises over the last 512 prefix positions
    tail = proj[8192 - 512:]
    assert tail[-64:].mean() > tail[:64].mean() + 2.0


def test_ragged_and_permuted_pages():
    cfg = synth.small("c4_ragged_b8", prefix=None)
    cfg = synth.dataclasses.replace(cfg, ragged=(100, 900))
    c = synth.make_case(cfg)
    assert c.batch == 8
    assert np.all((c.prefix_len >= 100) & (c.prefix_len <= 900))
    used = c.page_table[c.page_table >= 0]
    assert len(np.unique(used)) == len(used) == c.k_cache.shape[0] // 16
    assert not np.array_equal(np.sort(used), used)  # not the identity order
    for b in range(8):
        n_pages = -(-c.seq_len(b) // 16)
        assert np.all(c.page_table[b, :n_pages] >= 0) and np.all(c.page_table[b, n_pages:] == -1)
        assert c.k[b] == synth.pct_round_half_up(int(c.prefix_len[b]), 5)
