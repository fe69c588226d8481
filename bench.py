#!/usr/bin/env python3
"""Benchmark of the BN254 G1 multi-scalar multiplication on one MI355X.

One step = one whole MSM (decompose + sort, pair-tree accumulate, running-sum
reduction, window combine) over the n = 2^16, c = 13, S = 8 workload: independent
random points P_i = r_i * G and uniform scalars below r, the shape of the pages'
measurements (aztec-packages PR #23738 "Real-hardware data", PR #23520
"Measurements"). Inputs are generated on the device before timing and stay resident.

Prints one JSON line: throughput in points/s (value), latency per MSM, the
accumulate kernel against the integer-multiply roofline, and the CPU oracle timed
on this host's cores on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MSM latency ms and points/sec at n=2^16,c=13; achieved int-VALU % of peak"

# Peak rate of 32x32->64-bit multiply-adds (v_mad_u64_u32) on MI355X: 256 CUs x 4 SIMDs
# x 16 lanes per clock (the 64-bit-result multiply issues at half the 32-lane rate of
# plain 32-bit ALU ops) x 2.4 GHz.
PEAK_MAD_PER_S = 256 * 4 * 16 * 2.4e9
MAD_PER_MUL = 8 * 8 * 2 + 8          # CIOS product on 8 x 32-bit limbs
MAD_PER_ADD = 6 * MAD_PER_MUL        # batched affine add: 5 products + 1 square
# The inverse (a binary-GCD inverse, of the safegcd class the pages use) is counted as
# 45 products: the cost that the pages' software profile implies for it (inversion
# about 47% of the accumulate at S = 8, aztec-packages PR #23732 / #23738).
MAD_PER_INV = 45 * MAD_PER_MUL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the HIP sources: hardware counters taken on another build do not apply."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "elliptic_curve_scalar_amd", "csrc", "*"))):
        if f.endswith((".hip", ".hpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def counter_record(kind: str, workload: str, S: int, affine_levels: int, src: str):
    """A hardware-counter figure for the batched-affine kernel from the committed
    summaries under profiles/: kind "traffic" (HBM bytes per launch from rocprofv3
    FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size) or "valu" (int-VALU
    issue %). None when no entry matches this workload, S, schedule and kernel source."""
    name = {"traffic": "k_level_hbm_traffic.md", "valu": "k_level_valu_counters.md"}[kind]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if not line.startswith(kind + ": "):
                continue
            rec = json.loads(line[len(kind) + 2:])
            if (rec["workload"], rec["S"], rec["affine_levels"], rec["src"]) == (
                    workload, S, affine_levels, src):
                return rec
    return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="n65536_c13")
    ap.add_argument("--S", type=int, default=None, help="override the workload's S")
    ap.add_argument("--affine-levels", type=int, default=None,
                    help="pair-tree levels done with batched affine adds (-1: all)")
    ap.add_argument("--sched", type=int, default=0,
                    help="accumulate schedule: 0 pair tree, 1 stream walker")
    ap.add_argument("--walker-state", type=int, default=1,
                    help="stream walker slot state: 1 device buffer, 0 private memory")
    ap.add_argument("--prefix-store", type=int, default=0,
                    help="pair-tree level slot state: 0 private, 1 LDS; +2 caches denominators")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="CPU seconds for the oracle baseline (0 disables it)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB on the device once: "
                         "a kernel of known traffic for scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from elliptic_curve_scalar_amd import msm as M
    from elliptic_curve_scalar_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = wl.generate(args.workload)
    n, c = w["n"], w["c"]
    S = args.S or w["S"]
    log(f"[bench] workload {args.workload} n={n} c={c} S={S}")
    k = torch.from_numpy(w["dlogs"]).to(dev)
    scalars = torch.from_numpy(w["scalars"]).to(dev)
    points = M.g1_from_scalars(k)
    torch.cuda.synchronize()
    del k

    ctx = M.context(dev)
    if args.affine_levels is not None:
        ctx.set_affine_levels(args.affine_levels)
    ctx.set_walker_state(args.walker_state)
    ctx.set_prefix_store(args.prefix_store)
    out = torch.empty(16, dtype=torch.uint32, device=dev)
    for _ in range(args.warmup):
        ctx.run(points, scalars, c, S, out=out, sched=args.sched)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup})")

    # The timed steps bracket only the batched-affine kernel with events (its roofline);
    # the per-phase breakdown comes from separate, untimed steps afterwards.
    ctx.set_timing(1)
    ctx.timing_read()
    lat = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ts = time.perf_counter()
        ctx.run(points, scalars, c, S, out=out, sched=args.sched)
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - ts) * 1e3)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tm = ctx.timing_read()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ctx.set_timing(2)
    for _ in range(3):
        ctx.run(points, scalars, c, S, out=out, sched=args.sched)
    torch.cuda.synchronize()
    tm_phases = ctx.timing_read()
    ctx.set_timing(0)
    gpu_out = out.cpu().numpy().astype(np.uint32)
    if args.copy_mb > 0:
        src = torch.ones(args.copy_mb << 18, dtype=torch.int32, device=dev)
        dst = src.clone()
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    runs = max(1, tm["runs"])
    launches = max(1, tm["level_launches"])
    mads = tm["level_pairs"] * MAD_PER_ADD + tm["level_lanes"] * MAD_PER_INV
    level_s = tm["level_kernel_ms"] * 1e-3
    achieved = mads / level_s if level_s > 0 else 0.0
    al = args.affine_levels if args.affine_levels is not None else 1
    src = kernel_source_hash()
    tr = counter_record("traffic", args.workload, S, al, src)
    vu = counter_record("valu", args.workload, S, al, src)
    roofline = {
        "bound": "alu",
        "kernel": f"k_level<{S}> (pair-tree batched-affine accumulate)",
        "achieved": achieved / 1e12,
        "peak": PEAK_MAD_PER_S / 1e12,
        "unit": "TOP/s",
        "op": "32x32->64-bit multiply-add (algorithmic count)",
        "frac": achieved / PEAK_MAD_PER_S,
        "traffic": tr["bytes_per_launch"] if tr else None,
        "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
        "int_valu_pct": vu["int_valu_pct"] if vu else None,
        "launches_per_step": tm["level_launches"] / runs,
        "avg_launch_ms": tm["level_kernel_ms"] / launches,
        "algorithmic_ops_per_launch": mads / launches,
    }
    # per-phase times (events around every phase, from 3 untimed steps)
    phases = {kk: tm_phases[kk] / max(1, tm_phases["runs"])
              for kk in ("sort_ms", "accumulate_ms", "level_kernel_ms", "xyzz_level_ms",
                         "reduce_ms", "final_ms")}

    cpu = None
    verified = None
    if args.cpu_budget_s > 0:
        import oracle
        pts_host = oracle.g1_from_scalars(w["dlogs"])
        nthreads = min(oracle.num_windows(c), oracle.threads_default())
        times = []
        t_start = time.perf_counter()
        want = None
        while True:
            ts = time.perf_counter()
            want = oracle.msm_pippenger(pts_host, w["scalars"], c, threads=nthreads)
            times.append(time.perf_counter() - ts)
            if time.perf_counter() - t_start > args.cpu_budget_s or len(times) >= 50:
                break
        med = statistics.median(times)
        verified = bool(np.array_equal(gpu_out, want))
        cpu = {"value": n / med, "unit": "points/s", "cores": nthreads, "kind": "oracle",
               "sample": f"the full workload (n={n}, c={c}) run {len(times)} times; median "
                         f"{med * 1e3:.1f} ms per MSM",
               "ms_per_msm": med * 1e3}
        log(f"[bench] oracle: {med * 1e3:.1f} ms/MSM on {nthreads} threads; verified={verified}")

    rec = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": f"BN254 G1 MSM, n={n}, c={c}, S={S}, independent random points "
                               f"r_i*G, scalars uniform in [0, r) ({args.workload})",
                   "n": n, "c": c, "S": S, "sched": ["pair_tree", "walker"][args.sched],
                   "prefix_store": args.prefix_store, "walker_state": args.walker_state},
        "latency_ms": {"median": statistics.median(lat), "min": min(lat)},
        "phases_ms_per_step": phases,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "verified_vs_oracle": verified,
        "workspace_bytes": M.workspace_bytes(n, c, S),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
