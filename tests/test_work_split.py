"""Work split of the attention kernels, checked on the CPU.

The index math that maps a workgroup to its pieces of the (sequence, KV head)
key lists, and the combine kernel's lookup of a segment's partials, are
__host__ __device__ functions in csrc/attn_common.h.  A host build of them
(tests/host/work_split_main.hip) enumerates every piece; this test compares
the pieces with a direct model of the split (tile t of the concatenated lists
belongs to workgroup w iff floor(w T / W) <= t < floor((w + 1) T / W)) and
checks coverage, distinct partial indices, and the combine's lookup.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "work_split_main.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("ws") / "work_split")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "verification_guided_sparse_amd", "csrc"), SRC, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


def run(exe, mode, lens, Hkv, tile, W, split_tokens=0, splits=0):
    inp = f"{mode} {len(lens)} {Hkv} {tile} {W} {split_tokens} {splits} " + " ".join(map(str, lens))
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    pieces, comb = [], {}
    for line in out.splitlines():
        f = line.split()
        if f[0] == "P":
            pieces.append(tuple(int(x) for x in f[1:]))
        else:
            b, g, first, count = (int(x) for x in f[1:5])
            comb[(b, g)] = (first, count, [int(x) for x in f[5:]])
    return pieces, comb


def model_stream_k(lens, Hkv, tile, W):
    """Pieces (w, b, g, part, e_begin, e_end) straight from the definition."""
    owner = []  # tile of the concatenation -> (b, g, k): sequence-major, then KV head
    for b, L in enumerate(lens):
        for g in range(Hkv):
            owner += [(b, g, k) for k in range(-(-L // tile))]
    T = len(owner)
    out = []
    for w in range(W):
        runs = []  # [b, g, first k, last k] per maximal run of one segment
        for t in range(w * T // W, (w + 1) * T // W):
            b, g, k = owner[t]
            if runs and runs[-1][:2] == [b, g]:
                runs[-1][3] = k
            else:
                runs.append([b, g, k, k])
        out += [(w, b, g, w + b * Hkv + g, k0 * tile, min(lens[b], (k1 + 1) * tile))
                for b, g, k0, k1 in runs]
    return out


CASES = [
    ([100, 40], 2, 32, 3),
    ([1] * 37, 1, 32, 5),
    ([1] * 37, 8, 64, 256),
    ([1, 100000, 3, 7], 8, 32, 256),
    ([5000, 5000, 5000], 8, 32, 512),
    ([61387, 42705, 130832, 54734, 56543, 130158, 95835, 16774], 8, 32, 256),  # ragged batch of 8
    ([131079], 8, 32, 256),
    ([65542] * 4, 8, 32, 256),
    ([33, 1, 17], 2, 64, 1),
    ([200, 300], 4, 32, 1000),  # more workgroups than tiles
]


@pytest.mark.parametrize("lens,Hkv,tile,W", CASES)
def test_stream_k_pieces(harness, lens, Hkv, tile, W):
    pieces, comb = run(harness, 0, lens, Hkv, tile, W)
    assert pieces == model_stream_k(lens, Hkv, tile, W)
    parts = [p[3] for p in pieces]
    assert len(set(parts)) == len(parts) and max(parts) < W + len(lens) * Hkv
    for b, L in enumerate(lens):
        for g in range(Hkv):
            mine = sorted((p[4], p[5], p[0]) for p in pieces if (p[1], p[2]) == (b, g))
            assert mine[0][0] == 0 and mine[-1][1] == L
            assert all(x[1] == y[0] for x, y in zip(mine, mine[1:]))
            first, count, meets = comb[(b, g)]
            found = [first + j - (b * Hkv + g) for j in range(count) if meets[j]]
            assert found == [w for _, _, w in mine]


def test_stream_k_random(harness):
    rng = np.random.default_rng(7)
    for _ in range(25):
        B = int(rng.integers(1, 12))
        lens = [int(x) for x in rng.integers(1, 3000, B)]
        Hkv = int(rng.choice([1, 2, 4, 8]))
        tile = int(rng.choice([32, 64]))
        W = int(rng.integers(1, 600))
        pieces, comb = run(harness, 0, lens, Hkv, tile, W)
        assert pieces == model_stream_k(lens, Hkv, tile, W), (lens, Hkv, tile, W)


@pytest.mark.parametrize("lens,Hkv,split", [([5250], 8, 128), ([838, 6548, 10], 2, 128), ([7, 1], 4, 256),
                                             ([5250], 8, 165), ([3283] * 4, 8, 411), ([9, 40], 2, 13)])
def test_fixed_pieces(harness, lens, Hkv, split):
    splits = -(-max(lens) // split)
    W = len(lens) * Hkv * splits
    pieces, _ = run(harness, 1, lens, Hkv, 32, W, split, splits)
    assert len(pieces) == W
    for (w, b, g, part, e0, e1) in pieces:
        seg, sp = divmod(w, splits)
        assert (b, g, part) == (seg // Hkv, seg % Hkv, w)
        assert (e0, e1) == (min(lens[b], sp * split), min(lens[b], (sp + 1) * split))


@pytest.mark.parametrize("L,B,Hkv,tile,W", [(131079, 1, 8, 32, 256), (65542, 4, 8, 32, 256),
                                            (3001, 3, 8, 32, 40), (700, 16, 8, 32, 256),
                                            (5, 2, 4, 32, 1000), (64, 7, 2, 64, 9)])
def test_uniform_prefix_walk_matches_the_array_walk(harness, L, B, Hkv, tile, W):
    """With every list of the same length, the closed-form tile prefix (the
    kernels' speculation on equal lengths) gives exactly the pieces and
    combine lookups of the array prefix."""
    lens = [L] * B
    assert run(harness, 2, lens, Hkv, tile, W) == run(harness, 0, lens, Hkv, tile, W)
