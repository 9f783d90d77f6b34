"""Seeded synthetic inputs for one decode iteration of verification-guided sparse attention.

This module draws random tensors, adds the configured structure (an attention
sink, heavy-hitter keys, clustered spans of heavy hitters, a recency ramp),
rounds them once to the storage dtype, and lays the tokens out in a paged KV
cache.  It holds none of the method's arithmetic (no attention, aggregation or
selection): the oracle tests and the GPU path both consume the same host arrays
it returns, and neither side depends on the other.

Shapes are those of the attention layers the Vegas pages evaluate on (Qwen3-8B
and gpt-oss-20b, contexts up to 128K tokens; "Vegas" technical summary, section 4,
experimental results).  No dataset or model weight is used: every value is drawn
from a seeded generator.

Layouts (all C-contiguous host numpy arrays):
  q          [B][R][Hq][D]     R = gamma + 1 verify query rows
  q_draft    [gamma][B][Hq][D] one draft query per sequence and draft step
  k_cache    [num_pages * page_size][Hkv][D]   token-major paged cache
  v_cache    same as k_cache
  page_table [B][max_pages] int32, -1 past a sequence's last page
  prefix_len [B] int32          P_b; the R new tokens sit at positions P_b..P_b+gamma
  k          [B] int32          selection size per sequence
bf16 tensors are stored as their uint16 bit patterns; f32 tensors as float32.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16
_CHUNK = 1 << 22  # elements per independently seeded generator chunk


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  `k_pct` and `hh_pct` are integer percentages."""

    name: str
    batch: int
    prefix: tuple = ()          # per-sequence P_b (len == batch) unless `ragged`
    ragged: tuple | None = None  # (lo, hi): P_b drawn uniformly from [lo, hi]
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    dtype: str = "bf16"         # "bf16" or "f32"
    gamma: int = 4
    k_pct: int = 5
    sigma: float = 1.0
    hh_pct: int = 2             # heavy hitters as a percentage of P_b
    spans: int = 0              # number of clustered heavy-hitter spans
    span_len: int = 256
    sink: bool = True           # heavy-hitter direction added at position 0
    ramp: int = 0               # recency ramp length (0 = none)
    hh_scale: float = 3.0
    paging: str = "identity"    # "identity" or "permuted"
    page_size: int = PAGE_SIZE
    scale_mult: float = 1.0     # softmax scale = scale_mult / sqrt(D)
    seed: int = 0


# The five workloads: a small f32 case, then the Qwen3-8B- and gpt-oss-20b-shaped attention
# layers at 32K to 128K tokens of context.
CONFIGS: dict[str, Config] = {
    "c1_tiny": Config(
        name="c1_tiny", batch=1, prefix=(2048,), num_q_heads=8, num_kv_heads=2,
        head_dim=64, dtype="f32", gamma=4, k_pct=10, sigma=1.0 / 8.0, hh_pct=2,
        sink=True, ramp=0, paging="identity", seed=1000),
    "c2_qwen3_32k": Config(
        name="c2_qwen3_32k", batch=1, prefix=(32768,), gamma=4, k_pct=5,
        hh_pct=2, sink=True, ramp=512, seed=1001),
    "c3_qwen3_128k": Config(
        name="c3_qwen3_128k", batch=1, prefix=(131072,), gamma=6, k_pct=4,
        hh_pct=1, spans=3, span_len=256, sink=True, ramp=512, seed=1002),
    "c4_ragged_b8": Config(
        name="c4_ragged_b8", batch=8, ragged=(16384, 131072), gamma=4, k_pct=5,
        hh_pct=2, sink=True, ramp=512, paging="permuted", seed=1003),
    "c5_gptoss_64k": Config(
        name="c5_gptoss_64k", batch=4, prefix=(65536,) * 4, num_q_heads=64,
        num_kv_heads=8, head_dim=64, gamma=5, k_pct=5, hh_pct=2, sink=True,
        ramp=0, seed=1004),
}


def pct_round_half_up(n: int, pct: int) -> int:
    """n * pct / 100 rounded half up, in integer arithmetic."""
    return (n * pct + 50) // 100


@dataclass
class Case:
    cfg: Config
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    gamma: int
    page_size: int
    scale: float
    q: np.ndarray
    q_draft: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    page_table: np.ndarray
    prefix_len: np.ndarray
    k: np.ndarray
    heavy: list = field(default_factory=list)  # per sequence: sorted heavy-hitter positions

    @property
    def rows(self) -> int:
        return self.gamma + 1

    @property
    def max_prefix(self) -> int:
        return int(self.prefix_len.max())

    @property
    def max_k(self) -> int:
        return int(self.k.max())

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_slots(self) -> int:
        return int(self.k_cache.shape[0])

    def seq_len(self, b: int) -> int:
        """N_b: tokens in the cache for sequence b (prefix + the R new tokens)."""
        return int(self.prefix_len[b]) + self.rows


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    return max(1, min(8, os.cpu_count() or 1))


def _normal(seed: int, stream: tuple, n: int, sigma: float) -> np.ndarray:
    """n float32 draws of N(0, sigma^2).

    The flat array is cut into fixed-size chunks, each drawn from its own
    SeedSequence(seed, spawn_key=stream + (chunk,)), so the result does not depend
    on how many threads fill it.
    """
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // _CHUNK))

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        ss = np.random.SeedSequence(seed, spawn_key=tuple(stream) + (c,))
        g = np.random.Generator(np.random.PCG64(ss))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if sigma != 1.0:
            out[lo:hi] *= np.float32(sigma)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _rng(seed: int, stream: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(stream))))


def _unit_vectors(seed: int, b: int, hkv: int, d: int) -> np.ndarray:
    """One seeded unit direction per KV head, float32 [Hkv][D]."""
    u = _rng(seed, (3, b)).standard_normal((hkv, d)).astype(np.float64)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    return u.astype(np.float32)


def _heavy_positions(cfg: Config, seed: int, b: int, p: int) -> np.ndarray:
    """Sorted heavy-hitter positions in [1, p): `spans` clustered runs plus scattered ones."""
    if p == 0:
        return np.zeros(0, dtype=np.int64)
    n_hh = pct_round_half_up(p, cfg.hh_pct)
    g = _rng(seed, (4, b))
    taken = np.zeros(p, dtype=bool)
    taken[0] = True  # position 0 is the sink, handled separately
    chosen = []
    if cfg.spans > 0 and p > cfg.spans * cfg.span_len * 2:
        # non-overlapping spans: split [1, p) into `spans` equal bands, one span per band
        band = (p - 1) // cfg.spans
        for s in range(cfg.spans):
            lo = 1 + s * band
            start = lo + int(g.integers(0, band - cfg.span_len))
            chosen.append(np.arange(start, start + cfg.span_len))
            taken[start:start + cfg.span_len] = True
    n_scatter = max(0, n_hh - sum(len(c) for c in chosen))
    free = np.flatnonzero(~taken)
    if n_scatter > 0 and len(free) > 0:
        chosen.append(g.choice(free, size=min(n_scatter, len(free)), replace=False))
    if not chosen:
        return np.zeros(0, dtype=np.int64)
    return np.sort(np.concatenate(chosen).astype(np.int64))


def _prefix_lengths(cfg: Config, seed: int) -> np.ndarray:
    if cfg.ragged is not None:
        lo, hi = cfg.ragged
        return _rng(seed, (1,)).integers(lo, hi + 1, size=cfg.batch).astype(np.int32)
    assert len(cfg.prefix) == cfg.batch, "prefix must list one length per sequence"
    return np.asarray(cfg.prefix, dtype=np.int32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make_case(cfg: Config | str, seed: int | None = None) -> Case:
    """Build the seeded inputs of one workload (host arrays, see module docstring)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    B, Hq, Hkv, D = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    R = cfg.gamma + 1
    ps = cfg.page_size
    prefix = _prefix_lengths(cfg, seed)
    seq_len = prefix.astype(np.int64) + R
    npages = (seq_len + ps - 1) // ps
    total_pages = int(npages.sum())
    max_pages = int(npages.max())

    # physical page of each sequence's logical page
    if cfg.paging == "identity":
        phys = np.arange(total_pages, dtype=np.int64)
    elif cfg.paging == "permuted":
        phys = _rng(seed, (2,)).permutation(total_pages).astype(np.int64)
    else:
        raise ValueError(cfg.paging)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        page_table[b, : npages[b]] = phys[off: off + npages[b]]
        off += int(npages[b])

    num_slots = total_pages * ps
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    k_cache = np.zeros((num_slots, Hkv, D), dtype=sdt)
    v_cache = np.zeros((num_slots, Hkv, D), dtype=sdt)
    heavy = []
    for b in range(B):
        n = int(seq_len[b])
        p = int(prefix[b])
        kl = _normal(seed, (10, b), n * Hkv * D, cfg.sigma).reshape(n, Hkv, D)
        vl = _normal(seed, (11, b), n * Hkv * D, cfg.sigma).reshape(n, Hkv, D)
        u = _unit_vectors(seed, b, Hkv, D)
        hpos = _heavy_positions(cfg, seed, b, p)
        heavy.append(hpos)
        if cfg.sink and p > 0:
            kl[0] += np.float32(cfg.hh_scale) * u
        if len(hpos):
            kl[hpos] += np.float32(cfg.hh_scale) * u[None]
        if cfg.ramp > 0 and p > 0:
            r = min(cfg.ramp, p)
            j = np.arange(p - r, p)
            w = (cfg.hh_scale * (j - (p - r) + 1) / r).astype(np.float32)
            kl[p - r: p] += w[:, None, None] * u[None]
        # scatter logical tokens into physical slots
        pos = np.arange(n, dtype=np.int64)
        slots = page_table[b, pos // ps].astype(np.int64) * ps + pos % ps
        k_cache[slots] = _store(kl, cfg.dtype)
        v_cache[slots] = _store(vl, cfg.dtype)
        del kl, vl

    q = _store(_normal(seed, (20,), B * R * Hq * D, cfg.sigma).reshape(B, R, Hq, D), cfg.dtype)
    q_draft = _store(
        _normal(seed, (21,), cfg.gamma * B * Hq * D, cfg.sigma).reshape(cfg.gamma, B, Hq, D),
        cfg.dtype)
    k = np.array([pct_round_half_up(int(p), cfg.k_pct) for p in prefix], dtype=np.int32)
    scale = float(np.float32(cfg.scale_mult / math.sqrt(D)))
    return Case(cfg=cfg, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                dtype=cfg.dtype, gamma=cfg.gamma, page_size=ps, scale=scale, q=q,
                q_draft=q_draft, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
                prefix_len=prefix, k=k, heavy=heavy)


def with_k_pct(case: Case, k_pct: int) -> Case:
    """The same inputs with another selection budget k_b = round-half-up(P_b * k_pct / 100)."""
    k = np.array([pct_round_half_up(int(p), k_pct) for p in case.prefix_len], dtype=np.int32)
    return dataclasses.replace(case, cfg=dataclasses.replace(case.cfg, k_pct=k_pct), k=k)


def new_token_rows(case: Case, it: int) -> tuple[np.ndarray, np.ndarray]:
    """Seeded K/V rows of one iteration's gamma + 1 new tokens, [B][R][Hkv][D] in the
    case's storage dtype (same scale as the cache, no heavy-hitter terms)."""
    B, R, Hkv, D = case.batch, case.rows, case.num_kv_heads, case.head_dim
    n = B * R * Hkv * D
    k = _normal(case.cfg.seed, (30, it), n, case.cfg.sigma).reshape(B, R, Hkv, D)
    v = _normal(case.cfg.seed, (31, it), n, case.cfg.sigma).reshape(B, R, Hkv, D)
    return _store(k, case.dtype), _store(v, case.dtype)


def accepted_counts(case: Case, it: int) -> np.ndarray:
    """Seeded accepted-draft counts of one iteration, int32 [B] uniform in [0, gamma]."""
    return _rng(case.cfg.seed, (32, it)).integers(0, case.gamma + 1, case.batch).astype(np.int32)


def small(name: str, prefix=None, **kw) -> Config:
    """A shrunken copy of a named workload (same structure) for quick tests."""
    base = CONFIGS[name]
    if prefix is not None:
        kw["prefix"] = tuple(prefix)
        kw["batch"] = len(prefix)
        kw["ragged"] = None
    return dataclasses.replace(base, **kw)


def sharp(cfg: Config) -> Config:
    """Unit-scale data with a 4x softmax scale, so that a few keys dominate each row."""
    return dataclasses.replace(cfg, name=cfg.name + "_sharp", sigma=1.0, scale_mult=4.0)
