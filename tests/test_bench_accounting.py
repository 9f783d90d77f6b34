"""The benchmark's byte accounting and its one-GPU contract, checked on the CPU.

`bench.algorithmic_bytes` prices one layer iteration: the K/V rows each step
must read, the query and output rows, the exported logits and the selection's
score and index traffic.  The reference figures below are the per-workload
byte counts of the measurement plan (verify K+V, Q + out, group-sum export,
scores, draft step), each rounded there to the digits kept here; the test
compares within that rounding, so it pins the accounting to numbers worked
out independently of `bench.py`.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from verification_guided_sparse_amd import synth  # noqa: E402

MB = 1e6

# workload: (verify K+V MB, Q + out MB, group export MB, scores MB, draft step MB,
#            rounding of the K+V / draft figures in MB)
PLAN = {
    "c1_tiny": (2.10, 0.020, 0.016, 0.008, 0.21, 0.005),
    "c2_qwen3_32k": (134.2, 0.123, 1.05, 0.13, 6.71, 0.05),
    "c3_qwen3_128k": (536.9, 0.172, 4.19, 0.52, 21.5, 0.05),
    "c5_gptoss_64k": (536.9, 0.590, 8.39, 1.05, 26.8, 0.05),
}


@pytest.mark.parametrize("name", list(PLAN))
def test_algorithmic_bytes_match_the_plan(name):
    kv, qo, grp, sc, draft, tol = PLAN[name]
    c = synth.make_case(synth.CONFIGS[name])
    ab = bench.algorithmic_bytes(c, "group")
    # verify call = K+V + Q/out + the group-sum export it writes
    assert abs(ab["verify"] / MB - (kv + qo + grp)) <= tol + 0.01 * (qo + grp) + 0.005
    # aggregation reads the export and writes the scores
    assert abs(ab["aggregate"] / MB - (grp + sc)) <= 0.01 * (grp + sc) + 0.005
    # top-k reads the scores and writes k positions and slots (4 B each)
    k = int(c.k.sum())
    assert abs(ab["topk"] / MB - (sc + 8 * k / MB)) <= 0.01 * sc + 0.005
    # every draft step reads the selection's K/V rows (the plan's figure); the
    # causal tail (at most gamma entries) and the query/output rows add up to
    # 4 % at C1's 205-entry selection, far less at the others
    assert len(ab["draft"]) == c.gamma
    for s, d in enumerate(ab["draft"]):
        assert draft - tol <= d / MB <= draft + tol + 0.05 * draft, (s, d)
    assert ab["total"] == ab["verify"] + ab["aggregate"] + ab["topk"] + sum(ab["draft"])


def test_raw_export_adds_the_two_rows_of_every_head():
    """Raw logits: 2 rows x Hq heads x P x 4 B written and read back (33.6 MB
    each way at C3), against the group sums' Hkv x P x 4 B."""
    c = synth.make_case(synth.CONFIGS["c3_qwen3_128k"])
    raw, grp = bench.algorithmic_bytes(c, "raw"), bench.algorithmic_bytes(c, "group")
    assert abs((raw["verify"] - grp["verify"]) / MB - (33.6 - 4.19)) < 0.05
    assert abs((raw["aggregate"] - grp["aggregate"]) / MB - (33.6 - 4.19)) < 0.05


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr


def test_workload_figures_from_segment_times():
    """The per-workload figures divide the plan's bytes by the in-step segment
    times: verify call bytes over the verify segment per layer, the mean draft
    step's bytes over the draft segment per (step, layer), and the selection
    overhead as (verify+select - verify without export) / verify without export."""
    c = synth.make_case(synth.CONFIGS["c3_qwen3_128k"])
    ab = bench.algorithmic_bytes(c, "group")
    r = {"ms_per_step": 6.4, "layers": 36, "verify_us": 100.0, "draft_us": 10.0,
         "verify_select_us": 110.0, "verify_no_export_us": 100.0, "overhead_frac": 0.1}
    f = bench.workload_figures(c, r, "group")
    assert f["us_per_iter"] == round(6400 / 36, 2)
    assert f["verify_frac_in_step"] == round(ab["verify"] / 100e-6 / 1e9 / 8000, 4)
    draft_mean = sum(ab["draft"]) / len(ab["draft"])
    assert f["draft_frac_in_step"] == round(draft_mean / 10e-6 / 1e9 / 8000, 4)
    assert f["overhead_frac"] == 0.1


def test_percentiles_of_step_times():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0]
    assert bench.pct(xs, 50) == 3.0 and bench.pct(xs, 10) == 1.4 and bench.pct(xs, 90) == 4.6
