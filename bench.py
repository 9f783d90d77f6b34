"""Benchmark of the vegas_attn hot path on one MI355X.

A step is one Vegas decode iteration of the attention work of an L-layer
stack of the configured layer (default: the Qwen3-8B-shaped layer at 128K
context, gamma = 6, k = 4% of the prefix):

    for s in 0..gamma-1:  for each layer: sparse draft attention (draft step s)
    for each layer:       verify attention with the group-sum export,
                          aggregation and exact top-k (one vg_verify_select call)

Each layer has its own KV cache copy in HBM, so no layer's data is still in
the 256 MB MALL when it is read again: every byte counted below is an HBM
byte.  Inputs are seeded synthetic tensors, resident in HBM before timing.

Timing: the draft steps of all layers are one HIP graph and the verify calls
another; a timed step replays the two back to back on one stream, with HIP
events before, between and after them, so every step gives its own duration
and its two segments' durations.  Two more timed loops of the same shape
measure, in the same place in the step, the verify call on its own (then the
selection call) and the verify call without export: they give the verify
call's in-step duration (the roofline's dominant kernel) and the selection's
overhead against verify.

Printed: one JSON line with the whole-step achieved HBM GB/s (algorithmic
bytes / mean step time), the step-time median / p10 / p90, per-layer us per
iteration, the in-step fractions of HBM peak of the verify call and of the
draft call, the selection overhead, per-workload figures for the other
configurations, and the fp64 CPU oracle timed on a bounded sample of the
same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Achieved HBM GB/s & us/iter, verify+select+sparse-draft attention at 128K ctx"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_traffic.json")


def algorithmic_bytes(c, export):
    """Bytes the method must move per layer iteration (measurement)."""
    s_kv = 2 if c.dtype == "bf16" else 4
    row = c.num_kv_heads * c.head_dim * s_kv  # one token, all KV heads, K or V
    N = c.prefix_len.astype(np.int64) + c.rows
    P = c.prefix_len.astype(np.int64)
    kk = np.minimum(c.k, c.prefix_len).astype(np.int64)
    q_bytes = c.batch * c.rows * c.num_q_heads * c.head_dim * s_kv
    out_bytes = c.batch * c.rows * c.num_q_heads * c.head_dim * 4
    exp_rows = c.num_kv_heads if export == "group" else 2 * c.num_q_heads
    export_bytes = int(P.sum()) * exp_rows * 4
    verify = int(N.sum()) * 2 * row + q_bytes + out_bytes + export_bytes
    aggregate = export_bytes + int(P.sum()) * 4
    topk = int(P.sum()) * 4 + int(kk.sum()) * 8
    draft = []
    for s in range(c.gamma):
        keys = int((kk + s + 1).sum())
        draft.append(keys * 2 * row + c.batch * c.num_q_heads * c.head_dim * (s_kv + 4))
    return dict(verify=verify, aggregate=aggregate, topk=topk, draft=draft,
                total=verify + aggregate + topk + sum(draft))


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "verification_guided_sparse_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel_hash):
    """HBM bytes per verify launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("kernel_hash") != kernel_hash:
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(c, export, nthreads, min_seconds=10.0):
    """The fp64 oracle on the host cores: whole layer iterations of the workload,
    repeated until at least min_seconds of work; returns (seconds per
    iteration, iterations)."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while True:
        out, logits, group, _ = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len,
                                              c.gamma, c.scale, nthreads=nthreads)
        s = oracle.aggregate(group if export == "group" else logits, c.prefix_len)
        pos, slot, cnt = oracle.topk(s, c.prefix_len, c.k, page_table=c.page_table)
        for st in range(c.gamma):
            oracle.sparse(np.ascontiguousarray(c.q_draft[st][:, None]), c.k_cache, c.v_cache,
                          c.page_table, pos, cnt, c.prefix_len, np.full(c.batch, st + 1, np.int32),
                          c.scale, nthreads=nthreads)
        n += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= min_seconds:
            return elapsed / n, n


def host_info():
    """CPU model and online CPU count of the host (for the CPU baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def build_layers(c, L, kernel, export="group"):
    """L layer copies of workload c, each with its own KV cache in HBM, and one
    eager iteration each (the first draft step needs a selection)."""
    import torch
    from verification_guided_sparse_amd.runner import DeviceCase
    dev = torch.device("cuda:0")
    layers = [DeviceCase(c, device=dev, kernel=kernel)]
    for _ in range(L - 1):
        layers.append(DeviceCase(c, device=dev, kernel=kernel, like=layers[0]))
    for lc in layers:
        lc.iteration(export=export)
    torch.cuda.synchronize()
    return layers


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def segment_loop(graphs, steps):
    """Replays the graphs in order, `steps` times, on the current stream with a
    HIP event before, between and after them; returns per-step per-segment
    milliseconds ([steps][len(graphs)]) and the total milliseconds."""
    import torch
    n = len(graphs)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps * n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(steps):
        for i, g in enumerate(graphs):
            g.replay()
            ev[k * n + i + 1].record()
    torch.cuda.synchronize()
    seg = [[ev[k * n + i].elapsed_time(ev[k * n + i + 1]) for i in range(n)] for k in range(steps)]
    return seg, ev[0].elapsed_time(ev[steps * n])


def measure(c, layers, export, steps, warmup):
    """The timed step and the in-step segments of one workload (see the module
    docstring).  Durations in us per call (per layer), unless named _ms."""
    L, g = len(layers), max(c.gamma, 1)
    g_draft = capture(lambda: [lc.sparse(step=s) for s in range(c.gamma) for lc in layers])
    if export == "group":
        g_vsel = capture(lambda: [lc.verify_select() for lc in layers])
    else:
        g_vsel = capture(lambda: [(lc.verify(export=export), lc.select(src=export)) for lc in layers])
    g_verify = capture(lambda: [lc.verify(export=export) for lc in layers])
    g_select = capture(lambda: [lc.select(src=export) for lc in layers])
    g_none = capture(lambda: [lc.verify(export="none") for lc in layers])
    for _ in range(warmup):
        g_draft.replay()
        g_vsel.replay()
    t0 = time.perf_counter()
    seg, total_ms = segment_loop([g_draft, g_vsel], steps)  # the timed steps
    wall = time.perf_counter() - t0
    step_ms = [sum(x) for x in seg]
    seg_b, _ = segment_loop([g_draft, g_verify, g_select], steps)
    seg_c, _ = segment_loop([g_draft, g_none], steps)
    us = lambda xs, n: 1e3 * float(np.mean(xs)) / n
    r = {
        "ms_per_step": total_ms / steps,
        "step_ms_median": pct(step_ms, 50), "step_ms_p10": pct(step_ms, 10), "step_ms_p90": pct(step_ms, 90),
        "draft_us": us([x[0] for x in seg], g * L),
        "verify_select_us": us([x[1] for x in seg], L),
        "verify_us": us([x[1] for x in seg_b], L),
        "verify_us_p10": 1e3 * pct([x[1] for x in seg_b], 10) / L,
        "verify_us_p90": 1e3 * pct([x[1] for x in seg_b], 90) / L,
        "select_us": us([x[2] for x in seg_b], L),
        "verify_no_export_us": us([x[1] for x in seg_c], L),
        "wall_s_timed": wall,
    }
    r["overhead_frac"] = (r["verify_select_us"] - r["verify_no_export_us"]) / r["verify_no_export_us"]
    return r


def workload_figures(c, r, export):
    """Per-layer figures and fractions of the HBM peak from measure()'s result."""
    ab = algorithmic_bytes(c, export)
    draft_bytes = float(np.mean(ab["draft"])) if ab["draft"] else 0.0
    verify_gbs = ab["verify"] / (r["verify_us"] * 1e-6) / 1e9
    draft_gbs = draft_bytes / (r["draft_us"] * 1e-6) / 1e9 if r["draft_us"] > 0 else 0.0
    return {
        "us_per_iter": round(1e3 * r["ms_per_step"] / r["layers"], 2),
        "verify_us_in_step": round(r["verify_us"], 2),
        "verify_frac_in_step": round(verify_gbs / PEAK_HBM_GBS, 4),
        "draft_us_in_step": round(r["draft_us"], 2),
        "draft_frac_in_step": round(draft_gbs / PEAK_HBM_GBS, 4),
        "verify_select_us_in_step": round(r["verify_select_us"], 2),
        "verify_no_export_us_in_step": round(r["verify_no_export_us"], 2),
        "overhead_frac": round(r["overhead_frac"], 4),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3_qwen3_128k")
    ap.add_argument("--layers", type=int, default=0, help="layer copies (0: enough to exceed the MALL)")
    ap.add_argument("--export", choices=["group", "raw"], default="group")
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-workload figures of the other configurations")
    ap.add_argument("--other-workloads", default="c2_qwen3_32k,c4_ragged_b8,c5_gptoss_64k")
    ap.add_argument("--breakdown", action="store_true", help="also time every call kind separately")
    ap.add_argument("--collection", action="store_true",
                    help="also time the logit export + aggregation for two rows (Collect-2-Query) "
                         "against every row (full collection)")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the kernel-cost sweep over the selection ratio x gamma "
                         "(us per layer iteration at each point) for --workload")
    ap.add_argument("--sweep-gammas", default="2,4,6,8")
    ap.add_argument("--sweep-k-pcts", default="1,2,4,8,16")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (HBM byte-counter calibration)")
    ap.add_argument("--verify-replays", type=int, default=0, metavar="N",
                    help="only replay the verify calls (group export) of all layers N times and exit "
                         "(for HBM byte counters of the verify call)")
    ap.add_argument("--cpu-steps", default="", metavar="WORKLOADS",
                    help="only time the fp64 oracle's steps for these workloads (comma-separated) "
                         "on min(16, host CPUs) threads, and for the 2K and 32K ones also on one "
                         "thread (no GPU use)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.cpu_steps:
        wls = [w for w in args.cpu_steps.split(",") if w]
        cpu_steps(wls, [min(16, host_info()[1])])
        cpu_steps([w for w in wls if w in ("c1_tiny", "c2_qwen3_32k")], [1])
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path runs on a single MI355X and has no "
              "multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from verification_guided_sparse_amd import _binding as vg
    from verification_guided_sparse_amd import synth
    from verification_guided_sparse_amd.runner import V_CACHE_OFFSET

    vg.lib()  # fail loudly if the HIP library is missing
    if args.sweep:
        sweep(args)
        return
    kernel = {"auto": vg.VG_KERNEL_AUTO, "valu": vg.VG_KERNEL_VALU, "mfma": vg.VG_KERNEL_MFMA}[args.kernel]
    c = synth.make_case(args.workload)
    ab = algorithmic_bytes(c, args.export)
    L, layer_kv = layer_count(c, ab)
    if args.layers:
        L = args.layers
    print(f"[bench] {args.workload}: {L} layers, {layer_kv / 1e6:.1f} MB KV per layer, "
          f"export={args.export}, kernel={args.kernel}", file=sys.stderr, flush=True)
    layers = build_layers(c, L, kernel, args.export)
    if args.verify_replays:
        g_verify = capture(lambda: [lc.verify(export=args.export) for lc in layers])
        for _ in range(args.verify_replays):
            g_verify.replay()
        torch.cuda.synchronize()
        print(json.dumps({"verify_replays": args.verify_replays, "layers": L, "workload": args.workload,
                          "algorithmic_bytes_per_launch": ab["verify"]}), flush=True)
        return
    r = measure(c, layers, args.export, args.steps, args.warmup)
    r["layers"] = L
    fig = workload_figures(c, r, args.export)
    print(f"[bench] {args.workload}: {json.dumps(fig)}", file=sys.stderr, flush=True)

    bytes_per_step = ab["total"] * L
    value = bytes_per_step / (r["ms_per_step"] * 1e-3) / 1e9
    achieved = ab["verify"] / (r["verify_us"] * 1e-6) / 1e9
    traffic = measured_traffic(args.workload, kernel_source_hash())

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "batch": c.batch,
            "prefix": [int(x) for x in c.prefix_len] if c.batch <= 8 else int(c.max_prefix),
            "heads": f"{c.num_q_heads}q/{c.num_kv_heads}kv",
            "head_dim": c.head_dim,
            "gamma": c.gamma,
            "k": [int(x) for x in c.k],
            "layers_per_step": L,
            "export": args.export,
            "kernel": args.kernel,
            "v_cache_offset_bytes": V_CACHE_OFFSET,
            "parallelism": "single-gpu",
        },
        "step_ms": {"median": round(r["step_ms_median"], 4), "p10": round(r["step_ms_p10"], 4),
                    "p90": round(r["step_ms_p90"], 4)},
        "us_per_iter": fig["us_per_iter"],
        "roofline": {
            "kernel": "vg_verify_attention (attention kernel + its combine kernel), in-step",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "verify_us": round(r["verify_us"], 2),
            "verify_us_p10": round(r["verify_us_p10"], 2),
            "verify_us_p90": round(r["verify_us_p90"], 2),
            "algorithmic_bytes_per_launch": ab["verify"],
        },
        "targets": {
            "verify_frac_in_step": fig["verify_frac_in_step"],
            "draft_frac_in_step": fig["draft_frac_in_step"],
            "draft_us_in_step": fig["draft_us_in_step"],
            "overhead_frac": fig["overhead_frac"],
            "verify_select_us_in_step": fig["verify_select_us_in_step"],
            "verify_no_export_us_in_step": fig["verify_no_export_us_in_step"],
            "select_us_in_step_separate_call": round(r["select_us"], 2),
        },
        "wall_s_timed": round(r["wall_s_timed"], 3),
    }

    if args.breakdown:
        result["breakdown_us"] = breakdown(layers, c, args.export)
    if args.collection:
        result["collection_us"] = collection(layers)
    del layers
    torch.cuda.empty_cache()

    if not args.no_other_workloads:
        others = {}
        for wl in [w for w in args.other_workloads.split(",") if w and w != args.workload]:
            cw = synth.make_case(wl)
            Lw, _ = layer_count(cw, algorithmic_bytes(cw, args.export))
            lw = build_layers(cw, Lw, kernel, args.export)
            rw = measure(cw, lw, args.export, min(args.steps, 10), 2)
            rw["layers"] = Lw
            others[wl] = dict(workload_figures(cw, rw, args.export), layers=Lw)
            print(f"[bench] {wl}: {json.dumps(others[wl])}", file=sys.stderr, flush=True)
            del lw
            torch.cuda.empty_cache()
        result["other_workloads"] = others

    if not args.no_cpu_baseline:
        model, ncpu = host_info()
        nthreads = min(16, ncpu)  # the host's CPU share per GPU
        t, n_it = cpu_baseline(c, args.export, nthreads)
        result["cpu_baseline"] = {
            "value": round(ab["total"] / t / 1e9, 4),
            "unit": "GB/s",
            "cores": nthreads,
            "kind": "oracle",
            "sample": f"{n_it} full {args.workload} layer iterations (verify, aggregate, top-k, "
                      f"{c.gamma} draft steps) in fp64, {t:.2f} s each",
            "host_cpus": ncpu,
            "cpu_model": model,
        }
        c2 = synth.make_case("c2_qwen3_32k")
        t1, n1 = cpu_baseline(c2, args.export, 1, min_seconds=8.0)
        result["cpu_baseline_1thread"] = {
            "value": round(algorithmic_bytes(c2, args.export)["total"] / t1 / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{n1} full c2_qwen3_32k layer iterations in fp64 on one thread, {t1:.2f} s each",
        }
    print(json.dumps(result), flush=True)


def cpu_steps(workloads, threads):
    """The fp64 oracle's time per step (verify with the export, aggregation,
    top-k, one draft step) for each workload, on each thread count: one run of
    each step, wall clock."""
    import oracle
    from verification_guided_sparse_amd import synth
    model, ncpu = host_info()
    rows = []
    for wl in workloads:
        c = synth.make_case(wl)
        for nt in threads:
            t0 = time.perf_counter()
            out, logits, group, _ = oracle.verify(c.q, c.k_cache, c.v_cache, c.page_table, c.prefix_len,
                                                  c.gamma, c.scale, nthreads=nt)
            t1 = time.perf_counter()
            s = oracle.aggregate(group, c.prefix_len)
            t2 = time.perf_counter()
            pos, slot, cnt = oracle.topk(s, c.prefix_len, c.k, page_table=c.page_table)
            t3 = time.perf_counter()
            oracle.sparse(np.ascontiguousarray(c.q_draft[0][:, None]), c.k_cache, c.v_cache, c.page_table,
                          pos, cnt, c.prefix_len, np.full(c.batch, 1, np.int32), c.scale, nthreads=nt)
            t4 = time.perf_counter()
            row = {"workload": wl, "threads": nt, "verify_s": round(t1 - t0, 3),
                   "aggregate_ms": round(1e3 * (t2 - t1), 2), "topk_ms": round(1e3 * (t3 - t2), 2),
                   "draft_step_ms": round(1e3 * (t4 - t3), 2), "host_cpus": ncpu, "cpu_model": model}
            rows.append(row)
            print(json.dumps(row), flush=True)
    return rows


def calibrate_copy(nbytes):
    """Plain device-to-device copies of known size, for scaling the HBM byte
    counters read for the attention kernels: 3 launches of the runtime's copy
    kernel (dst.copy_) and 3 of an elementwise copy with 16-byte loads per lane
    (torch.mul by 1), which reads whole 128-byte lines like the attention kernels."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "launches": 3,
                      "kernels": ["runtime copy (dst.copy_)", "elementwise copy (torch.mul by 1)"]}), flush=True)


def capture(fn):
    """Record fn's launches into a HIP graph (torch.cuda.CUDAGraph on ROCm)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_graph_us(fn, n_layers, reps=5):
    """Per-layer us of fn (all layers' calls captured in one graph), HIP events."""
    import torch
    g = capture(fn)
    g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (reps * n_layers)


def collection(layers):
    """Cost of the logit export + aggregation with Collect-2-Query (rows 0 and gamma)
    and with full collection (every row), for the raw and the group export: each is
    verify-with-export minus verify-without-export, plus the aggregation of that
    export (per layer, us)."""
    n = len(layers)
    t = {
        "verify_none": timed_graph_us(lambda: [lc.verify(export="none") for lc in layers], n),
        "verify_raw_two": timed_graph_us(lambda: [lc.verify(export="raw") for lc in layers], n),
        "verify_raw_all": timed_graph_us(lambda: [lc.verify(export="raw", rows="all") for lc in layers], n),
        "verify_group_two": timed_graph_us(lambda: [lc.verify(export="group") for lc in layers], n),
        "verify_group_all": timed_graph_us(lambda: [lc.verify(export="group", rows="all") for lc in layers], n),
        "aggregate_raw_two": timed_graph_us(lambda: [lc.aggregate(src="raw") for lc in layers], n),
        "aggregate_raw_all": timed_graph_us(lambda: [lc.aggregate(src="raw_all") for lc in layers], n),
        "aggregate_group": timed_graph_us(lambda: [lc.aggregate(src="group") for lc in layers], n),
    }
    out = {k: round(v, 2) for k, v in t.items()}
    base = t["verify_none"]
    out["overhead_raw_two"] = round(t["verify_raw_two"] - base + t["aggregate_raw_two"], 2)
    out["overhead_raw_all"] = round(t["verify_raw_all"] - base + t["aggregate_raw_all"], 2)
    out["overhead_group_two"] = round(t["verify_group_two"] - base + t["aggregate_group"], 2)
    out["overhead_group_all"] = round(t["verify_group_all"] - base + t["aggregate_group"], 2)
    return out


def layer_count(c, ab):
    """Layer copies per timed step: enough draft bytes to exceed the 256 MB MALL
    three times over, at most 64 layers and 40 GB of KV."""
    layer_kv = int((c.prefix_len.astype(np.int64) + c.rows).sum()) * c.num_kv_heads * c.head_dim * 2 * (
        2 if c.dtype == "bf16" else 4)
    L = max(2, int(np.ceil(3 * 256e6 / max(sum(ab["draft"]) / max(c.gamma, 1), 1))))
    return min(L, 64, max(2, int(40e9 // layer_kv))), layer_kv


def sweep(args):
    """Kernel cost of one layer iteration over a grid of gamma x selection ratio
    (the cost half of the pages' tuning procedure: accepted-token rates need a
    model and are not measured).  Per point: the whole iteration (verify with
    export, aggregate, top-k, gamma draft steps) and its draft part, each over
    all layer copies in one HIP graph, HIP events."""
    import dataclasses
    import torch
    from verification_guided_sparse_amd import synth
    from verification_guided_sparse_amd.runner import DeviceCase
    gammas = [int(x) for x in args.sweep_gammas.split(",")]
    pcts = [int(x) for x in args.sweep_k_pcts.split(",")]
    base_cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    points = []
    for gamma in gammas:
        case = synth.make_case(dataclasses.replace(base_cfg, gamma=gamma))
        for pct in pcts:
            c = synth.with_k_pct(case, pct)
            L, _ = layer_count(c, algorithmic_bytes(c, args.export))
            layers = [DeviceCase(c, device=dev)]
            layers += [DeviceCase(c, device=dev, like=layers[0]) for _ in range(L - 1)]
            for lc in layers:
                lc.iteration(export=args.export)
            torch.cuda.synchronize()

            def it():
                for lc in layers:
                    if args.export == "group":
                        lc.verify_select()
                    else:
                        lc.verify(export=args.export)
                        lc.select(src=args.export)
                for s in range(c.gamma):
                    for lc in layers:
                        lc.sparse(step=s)

            def drafts():
                for s in range(c.gamma):
                    for lc in layers:
                        lc.sparse(step=s)

            us_it = timed_graph_us(it, L, reps=max(args.steps // 5, 3))
            us_dr = timed_graph_us(drafts, L, reps=max(args.steps // 5, 3))
            p = {"gamma": gamma, "k_pct": pct, "k": [int(x) for x in c.k], "layers": L,
                 "us_per_iter": round(us_it, 2), "us_verify_select": round(us_it - us_dr, 2),
                 "us_drafts": round(us_dr, 2), "us_per_draft_step": round(us_dr / max(gamma, 1), 2)}
            points.append(p)
            print(f"[sweep] {json.dumps(p)}", file=sys.stderr, flush=True)
            del layers
            torch.cuda.empty_cache()
    print(json.dumps({"sweep": args.workload, "export": args.export, "unit": "us per layer iteration",
                      "points": points}), flush=True)


def breakdown(layers, c, export):
    """Per-call durations: each call kind over all layers captured in its own graph,
    replayed and timed with HIP events; reported per call (us)."""
    import torch
    reps = 5
    kinds = {
        "verify": lambda: [lc.verify(export=export) for lc in layers],
        "verify_no_export": lambda: [lc.verify(export="none") for lc in layers],
        # verify, aggregation and top-k in one call (the step's form with the group export)
        "verify_select": lambda: [lc.verify_select() for lc in layers],
        # aggregation + top-k in one call
        "select": lambda: [lc.select(src=export) for lc in layers],
        # the same work as two calls: aggregation with the fused first radix pass, then top-k
        "aggregate": lambda: [lc.aggregate(src=export, fuse_prepass=True) for lc in layers],
        "topk_after_prepass": lambda: [lc.topk(prepass_done=True) for lc in layers],
        "draft": lambda: [lc.sparse(step=c.gamma - 1) for lc in layers],
        # rewrites the new tokens' own rows: the workload is unchanged
        "kv_append": lambda: [lc.append() for lc in layers],
        # the query-agnostic baseline: sink + recent window, then a draft step over it
        "window_select": lambda: [lc.window(n_sink=4) for lc in layers],
        "draft_over_window": lambda: [lc.sparse(step=c.gamma - 1) for lc in layers],
    }
    for lc in layers:
        lc.new_rows()  # allocated before capture
    out = {}
    for name, fn in kinds.items():
        if name == "topk_after_prepass":
            # the prepass must precede every top-k: time (aggregate + topk) and subtract
            g = capture(lambda: [(lc.aggregate(src=export, fuse_prepass=True), lc.topk(prepass_done=True))
                                 for lc in layers])
        else:
            g = capture(fn)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        out[name] = 1e3 * a.elapsed_time(b) / (reps * len(layers))
    out["topk"] = out.pop("topk_after_prepass") - out["aggregate"]
    out = {k: round(v, 2) for k, v in out.items()}
    # export + aggregation + top-k added to verify attention without export
    sel_path = out["verify_select"] if export == "group" else out["verify"] + out["select"]
    out["overhead_frac"] = round((sel_path - out["verify_no_export"]) / out["verify_no_export"], 4)
    g = max(c.gamma, 1)
    out["iteration_vegas"] = round(sel_path + g * out["draft"], 2)
    out["iteration_window"] = round(out["verify_no_export"] + out["window_select"] + g * out["draft_over_window"], 2)
    # restore a consistent selection for later replays
    for lc in layers:
        lc.iteration(export=export)
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    main()
